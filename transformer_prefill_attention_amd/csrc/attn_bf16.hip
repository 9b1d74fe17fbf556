// attn_bf16.hip -- causal grouped-query attention with bf16 MFMA inputs and f32
// accumulation (v_mfma_f32_32x32x16_bf16).
//
// Passages: as attn_f32.hip (memra-engine 0.130.0 src/forward.rs, SDPA block;
// memra-engine 0.101.0 src/spec.rs, `full_attn_verify` per-row fallback for the
// causal rule).  What is rounded to bf16 (round to nearest even): the scaled Q,
// K, V and the softmax weights P, each just before its product; the scores, the
// softmax, the accumulation and the output stay f32 (the denominator f64).
//
// Two kernels:
//  * stage_kv_bf16_kernel converts K and V once into a workspace of 64-key
//    tiles per (K/V head, sequence), each tile laid out byte for byte as the
//    attention kernel keeps it in LDS: K row-major with the 16-byte chunks of a
//    row XOR-swizzled by the row index, V transposed (V^T[d][key]) with the keys
//    of each row in MFMA operand order and the same kind of swizzle.  Rows past
//    the end of a sequence are zeros.  Without this step every workgroup would
//    convert every tile it visits again (about T/64 times per tile).
//  * attn_bf16_kernel: one workgroup of eight wavefronts per (K/V head, query
//    super-block), S^T = K Q^T so that P lands in the B-operand layout of
//    O^T += V^T P^T, online softmax in base 2 as in the f32 kernel.  Tiles move
//    HBM/L2 -> LDS with direct-to-LDS loads (no registers, no conversion).
//
// Ping-pong schedule.  Wavefronts 0-3 (group A) and 4-7 (group B) sit on the
// four SIMDs in pairs (one of each group per SIMD).  Each wavefront runs the
// same sequence of phases, matrix phase M(t) = [P(t-1) V(t-1), S(t) = K(t) Q^T]
// then softmax phase X(t) = [scores -> P(t)], with a workgroup barrier after
// every phase; group B starts one phase late.  So in every barrier interval one
// wavefront of each SIMD issues MFMAs while the other does the exponentials,
// and the softmax work hides behind the matrix cores instead of adding to them.
// The loads of K(t+1) and V(t) are issued in global phase 2t and waited for at
// the end of phase 2t+1; LDS holds two K and two V tiles.
//
// O is rescaled lazily: the running max used for the exponentials only moves
// when a new score exceeds it by more than 8 (log2 units), so P stays <= 256
// and, on typical data, O is rescaled only in the first tiles.  The softmax
// denominator adds up the bf16-rounded weights (v_dot2 against ones), the same
// numbers the P.V product uses.
//
// PREP = true is the fused entry (qk_prep_attn): the staging kernel RMS-normalises
// and rotates each K row before converting it (and can copy the rotated rows out
// for a cache), and the attention kernel does the same to its Q rows once, in its
// prologue.  The normalised Q and K never go to HBM except for that optional copy.
//
// Q8 = true reads an 8-bit store (needle-core v3/model.rs: a quantised session's int8
// K/V store, one scale per row; launch_attn_q8): Q arrives as codes and the softmax
// scale, log2(e) and the row's Q scale stay in one register qf.  With head_dim 128 the
// K tiles hold int8 codes and the scores come from v_mfma_i32_32x32x32_i8 (half the
// matrix-core time of the bf16 product, half the K tile bytes); with 64, codes sit in
// bf16 K tiles (exact) on the bf16 MFMA.  Either way the integer scores are exact.  The
// 64 key scales of a tile ride with its K tile into a ring of four LDS slots, and the X
// phase computes score = s_int * k_scale, weight = 2^(score * qf - m).  V tiles are
// dequantised by the staging kernel, so P.V is unchanged.
//
// SPLIT = true is the PFA_PREC_BF16X3 mode: Q and K are each split into a bf16
// high part and a bf16 low part (x = hi + lo to ~2^-17) and the scores take the
// three products hi.hi + hi.lo + lo.hi, so score rounding no longer grows with
// |score| the way plain bf16 inputs do (keys with large norms); P and V stay
// plain bf16.  The K tiles carry both parts.
#include "pfa_device.h"
#include "pfa_internal.h"

namespace pfa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx16 __attribute__((ext_vector_type(16)));

constexpr int kBN = kBf16TileKeys;  // keys per tile (64)
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));

// The 16-bit operands of the products: bf16, or with F16 IEEE binary16 (PFA_PREC_F16),
// whose bits sit in the same 2-byte slots (no tile layout depends on the format).  Both
// round to nearest even.
template <bool F16>
__device__ __forceinline__ __bf16 to16(float x) {
    if constexpr (F16) return __builtin_bit_cast(__bf16, (_Float16)x);
    else return (__bf16)x;
}
// Two at a time, as one packed conversion (binary16: v_cvt_pk_f16_f32, which rounds to
// nearest even; converting the two elements separately costs two conversions and a permute)
template <bool F16>
__device__ __forceinline__ bf16x2 to16x2(float a, float b) {
    if constexpr (F16) {
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(bf16x2, __builtin_convertvector(f32x2{a, b}, halfx2));
    } else {
        return bf16x2{(__bf16)a, (__bf16)b};
    }
}
template <bool F16>
__device__ __forceinline__ floatx16 mfma16(bf16x8 a, bf16x8 b, floatx16 c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a),
                                                      __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// acc + x[0] + x[1], the two weights as rounded for the P.V product
template <bool F16>
__device__ __forceinline__ float add_pair(bf16x2 x, float acc) {
    if constexpr (F16) {
        const halfx2 ones = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(halfx2, x), ones, acc, false);
    } else {
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(x, ones, acc, false);
    }
}

// Position of 16-byte chunk `c` in row `row` of an LDS tile with `nch` chunks per
// row.  Any 16 consecutive rows of a 32-row block map one logical chunk to 16
// different positions (and rows of equal parity to 8 different ones), so the
// ds_read_b128 of one chunk from 32 rows spreads over all banks.
__device__ __forceinline__ int swz(int row, int c, int nch) {
    return c ^ ((row % nch) ^ ((row / nch) & 1));
}

// Rotary table of the fused entry, after the K and V tiles in the workspace:
// (cos, sin) of position p and pair j at p * D/2 + j (pairs j >= rope_dim/2 unused).
template <int D, bool SPLIT>
__device__ __forceinline__ const float2* rope_table(const __bf16* ws, int Hkv, int n_tiles) {
    constexpr int KP = SPLIT ? 2 : 1;
    return reinterpret_cast<const float2*>(ws + (int64_t)Hkv * n_tiles * (KP + 1) * kBN * D);
}

// One entry per (position < rows, pair j < D/2), angle reduced in f64 (rope_cos_sin).
// A block covers kTabRows positions; thread t owns pair t % (D/2) (one pow each).
constexpr int kTabRows = 64;
template <int D, bool SPLIT>
__global__ __launch_bounds__(256) void rope_table_kernel(__bf16* ws, int Hkv, int n_tiles,
                                                         int rows, int n, double base) {
    float2* tab = const_cast<float2*>(rope_table<D, SPLIT>(ws, Hkv, n_tiles));
    constexpr int RPP = 256 / (D / 2);  // positions per pass
    const int j = threadIdx.x % (D / 2);
    const bool rot = 2 * j < n;
    const double turns = rot ? rope_turns_per_pos(j, n, base) : 0.0;
    const int p_end = min(rows, (int)(blockIdx.x + 1) * kTabRows);
    for (int pos = blockIdx.x * kTabRows + threadIdx.x / (D / 2); pos < p_end; pos += RPP) {
        float c = 1.0f, sn = 0.0f;
        if (rot) rope_cos_sin(pos, turns, c, sn);
        tab[(int64_t)pos * (D / 2) + j] = float2{c, sn};
    }
}

// V^T staging buffer of the staging kernels: D rows of kVts bf16 (the 4-key runs stay
// 8-byte aligned).  store_vt_rows writes its rows to a V tile: row d holds 8 groups of
// 8 keys, group p = 2s + h being keys 16s + 4h + {0..3} and 16s + 8 + 4h + {0..3} (the
// keys lane half h feeds at P.V step s), group p stored at position swz(d, p, 8).
constexpr int kVts = kBN + 8;
template <int D>
__device__ __forceinline__ void store_vt_rows(const __bf16* vts, __bf16* vt, int tid) {
#pragma unroll
    for (int i = 0; i < 8 * D / 256; ++i) {
        const int f = tid + 256 * i;
        const int d = f / 8, p = f % 8;
        const int s4 = p >> 1, h = p & 1;
        const bf16x4 lo4 = *reinterpret_cast<const bf16x4*>(vts + d * kVts + 16 * s4 + 4 * h);
        const bf16x4 hi4 = *reinterpret_cast<const bf16x4*>(vts + d * kVts + 16 * s4 + 8 + 4 * h);
        const bf16x8 x = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        *reinterpret_cast<bf16x8*>(vt + d * kBN + 8 * swz(d, p, 8)) = x;
    }
}

// One tile's rows of a 256-thread block, shared by the staging kernels.
// 8 dims (logical chunk c of row r) -> bf16 high (and low) parts at the swizzled place.
template <int D, bool SPLIT, bool F16>
__device__ __forceinline__ void store_k_chunk(__bf16* tile, int r, int c, const float* x) {
    static_assert(!(SPLIT && F16), "the split scores are a bf16 mode");
    constexpr int NCH = D / 8;
    bf16x8 hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        hi[e] = to16<F16>(x[e]);
        if constexpr (SPLIT) lo[e] = (__bf16)(x[e] - (float)hi[e]);
    }
    const int pos = swz(r, c, NCH);
    *reinterpret_cast<bf16x8*>(tile + r * D + 8 * pos) = hi;
    if constexpr (SPLIT) *reinterpret_cast<bf16x8*>(tile + kBN * D + r * D + 8 * pos) = lo;
}
// V rows 0 .. nval-1 (stride row_stride floats; zeros past nval) -> V^T in vts.  4 keys x
// 4 dims per block, loaded as 4 float4 rows, written as four 4-key runs of V^T.  Block b:
// dims 4 (b % (D/4)) .., keys 4 (b / (D/4)) ..
template <int D, bool F16>
__device__ __forceinline__ void stage_v_rows(const float* vin, int64_t row_stride, int nval,
                                             __bf16* vts, int tid) {
    constexpr int VB = kBN * D / 16;
#pragma unroll
    for (int i = 0; i < VB / 256; ++i) {
        const int b = tid + 256 * i;
        const int d0 = 4 * (b % (D / 4)), key0 = 4 * (b / (D / 4));
        floatx4 r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            r[e] = key0 + e < nval ? *reinterpret_cast<const floatx4*>(vin + (key0 + e) * row_stride + d0)
                                   : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            bf16x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = to16<F16>(r[e][c]);
            *reinterpret_cast<bf16x4*>(vts + (d0 + c) * kVts + key0) = x;
        }
    }
}
// K rows 0 .. nval-1 (zeros past nval) -> the K tile: 16-byte chunks (8 dims) of each
// row, converted and written to their swizzled place.
template <int D, bool SPLIT, bool F16>
__device__ __forceinline__ void stage_k_rows(const float* kin, int64_t row_stride, int nval,
                                             __bf16* kt, int tid) {
    constexpr int NCH = D / 8;
#pragma unroll
    for (int i = 0; i < kBN * NCH / 256; ++i) {
        const int f = tid + 256 * i;
        const int r = f / NCH, c = f % NCH;
        floatx4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
        if (r < nval) {
            const float* src = kin + r * row_stride + 8 * c;
            a = *reinterpret_cast<const floatx4*>(src);
            b = *reinterpret_cast<const floatx4*>(src + 4);
        }
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = e < 4 ? a[e] : b[e - 4];
        store_k_chunk<D, SPLIT, F16>(kt, r, c, x);
    }
}

// ---------------------------------------------------------------------------
// K/V -> bf16 tiles.  Block = (K/V head, tile over all sequences).
//  K tile: KP parts (high, low) x 64 rows x D; element (r, c) at r*D + 8*swz(r, c/8, D/8) + c%8.
//  V tile: D rows x 64 keys; row d holds 8 groups of 8 keys, group p = 2s + h being
//  keys 16s + 4h + {0..3} and 16s + 8 + 4h + {0..3} (the keys lane half h feeds
//  at P.V step s), group p stored at position swz(d, p, 8).
template <int D, bool SPLIT, bool PREP, bool F16>
__global__ __launch_bounds__(256) void stage_kv_bf16_kernel(const float* __restrict__ k,
                                                            const float* __restrict__ v,
                                                            __bf16* __restrict__ ws,
                                                            AttnSched sched, int Hkv,
                                                            PrepParams prep) {
    constexpr int KP = SPLIT ? 2 : 1;
    constexpr int KRS = D + 4;    // raw K row stride in LDS (f32), fused entry only
    __shared__ __attribute__((aligned(16))) __bf16 vts[D * kVts];
    __shared__ __attribute__((aligned(16))) float kraw[PREP ? kBN * KRS : 4];
    const int tid = threadIdx.x;
    const int kv = blockIdx.x % Hkv;
    const int gt = blockIdx.x / Hkv;
    const int n_tiles = sched.n_tiles;
    const int s = find_seq(sched.tile_off, sched.n_seqs, gt);
    const int k0 = sched.koff[s] + (gt - sched.tile_off[s]) * kBN;  // the tile's key rows
    const int nval = min(kBN, sched.koff[s + 1] - k0);
    const int64_t row_stride = (int64_t)Hkv * D;
    __bf16* kt = ws + ((int64_t)kv * n_tiles + gt) * (KP * kBN * D);
    __bf16* vt = ws + (int64_t)Hkv * n_tiles * (KP * kBN * D) +
                 ((int64_t)kv * n_tiles + gt) * (kBN * D);
    const float* kin = k + (int64_t)k0 * row_stride + kv * D;
    const float* vin = v + (int64_t)k0 * row_stride + kv * D;
    stage_v_rows<D, F16>(vin, row_stride, nval, vts, tid);
    if constexpr (!PREP) {
        stage_k_rows<D, SPLIT, F16>(kin, row_stride, nval, kt, tid);
    } else {
        // Fused entry: RMS-normalise and rotate each K row on its way in.  Four threads
        // per row take D/4 consecutive dims each.  A rotation partner (dim c +- n/2) sits
        // in the quarter two apart when n = D and one apart when n = D/2 (DPP quad
        // permutations); any other rope_dim goes through LDS.  Rows past the sequence
        // end are zeros.
        const int n = prep.rope_dim, half = n >> 1;
        const float2* tab = rope_table<D, SPLIT>(ws, Hkv, n_tiles);
        constexpr int DQ = D / 4;  // dims per thread
        const int r = tid >> 2, qd = tid & 3, c0 = qd * DQ;
        const bool valid = r < nval;
        const int pos = valid ? k0 + r - sched.koff[s] : 0;  // rows past the end: any valid entry
        float y[DQ];
#pragma unroll
        for (int i = 0; i < DQ; i += 4) {
            const floatx4 x = valid ? *reinterpret_cast<const floatx4*>(kin + r * row_stride + c0 + i)
                                    : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) y[i + e] = x[e];
        }
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < DQ; ++i) ss += y[i] * y[i];
        ss += dpp_f32<0xB1>(ss);  // quad_perm [1,0,3,2]
        ss += dpp_f32<0x4E>(ss);  // quad_perm [2,3,0,1]
        const float rs = 1.0f / sqrtf(ss * (1.0f / D) + prep.eps);
#pragma unroll
        for (int i = 0; i < DQ; i += 4) {
            const floatx4 w = *reinterpret_cast<const floatx4*>(prep.wk + c0 + i);
#pragma unroll
            for (int e = 0; e < 4; ++e) y[i + e] *= rs * w[e];
        }
        const float2* trow = tab + pos * (D / 2);
        if (n == D || n == D / 2) {
            // partner quarter: qd ^ 2 (n = D) or qd ^ 1 (n = D/2, quarters 0 and 1 only)
            const bool full = n == D;
            const bool first = full ? qd < 2 : qd == 0;  // holds the pair's first dims
            const bool rot = full || qd < 2;
            // (cos, sin) of two pairs per 16-byte load (table rows start on 16-byte
            // boundaries)
            const floatx4* tj = reinterpret_cast<const floatx4*>(trow + (full ? (qd & 1) * DQ : 0));
#pragma unroll
            for (int i = 0; i < DQ; i += 2) {
                const floatx4 t2 = tj[i / 2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const float yp = full ? dpp_f32<0x4E>(y[i + u]) : dpp_f32<0xB1>(y[i + u]);
                    const float tc = t2[2 * u], ts = t2[2 * u + 1];
                    const float yr = first ? y[i + u] * tc - yp * ts : y[i + u] * tc + yp * ts;
                    y[i + u] = rot ? yr : y[i + u];
                }
            }
        } else {
            __syncthreads();  // (uniform: n is a kernel argument)
            float* xr = kraw + r * KRS;
#pragma unroll
            for (int i = 0; i < DQ; i += 4)
                *reinterpret_cast<floatx4*>(xr + c0 + i) = floatx4{y[i], y[i + 1], y[i + 2], y[i + 3]};
            __syncthreads();
#pragma unroll
            for (int i = 0; i < DQ; ++i) {
                const int c = c0 + i;
                if (c < n) {
                    const int j = c < half ? c : c - half;
                    const float yp = xr[c < half ? c + half : c - half];
                    const float2 t = trow[j];
                    y[i] = c < half ? y[i] * t.x - yp * t.y : y[i] * t.x + yp * t.y;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < DQ; ++i) y[i] = valid ? y[i] : 0.0f;
        if (prep.k_rot_out && valid) {
            float* dst = prep.k_rot_out + (int64_t)(k0 + r) * row_stride + kv * D + c0;
#pragma unroll
            for (int i = 0; i < DQ; i += 4)
                *reinterpret_cast<floatx4*>(dst + i) = floatx4{y[i], y[i + 1], y[i + 2], y[i + 3]};
        }
#pragma unroll
        for (int cc = 0; cc < DQ / 8; ++cc)
            store_k_chunk<D, SPLIT, F16>(kt, r, c0 / 8 + cc, y + 8 * cc);
    }
    __syncthreads();
    store_vt_rows<D>(vts, vt, tid);
}

// ---------------------------------------------------------------------------
// Kept tiles (TileAppend): block = (K/V head, touched tile).  The tile's rows are
// staged from the f32 cache as stage_kv_bf16_kernel stages them (rows past the
// sequence's end are zeros), into the tile's place in its sequence slot; the blocks of
// K/V head 0 also write the rotary-table rows of the tile's positions as
// rope_table_kernel computes them.
template <int D, bool SPLIT, bool F16>
__global__ __launch_bounds__(256) void append_tiles_kernel(const float* __restrict__ k,
                                                           const float* __restrict__ v,
                                                           __bf16* __restrict__ tiles,
                                                           TileAppend app, int Hkv) {
    constexpr int KP = SPLIT ? 2 : 1;
    __shared__ __attribute__((aligned(16))) __bf16 vts[D * kVts];
    const int tid = threadIdx.x;
    const int kv = blockIdx.x % Hkv;
    const int g = blockIdx.x / Hkv;
    const int s = find_seq(app.cum, app.n_seqs, g);
    const int lt = app.first[s] + (g - app.cum[s]);           // tile of the sequence
    const int k0 = app.koff[s] + lt * kBN;                     // its first cache row
    const int nval = min(kBN, app.koff[s + 1] - k0);
    const int n_tiles = app.n_seqs * app.cap_tiles;
    const int gt = s * app.cap_tiles + lt;
    const int64_t row_stride = (int64_t)Hkv * D;
    __bf16* kt = tiles + ((int64_t)kv * n_tiles + gt) * (KP * kBN * D);
    __bf16* vt = tiles + (int64_t)Hkv * n_tiles * (KP * kBN * D) +
                 ((int64_t)kv * n_tiles + gt) * (kBN * D);
    stage_v_rows<D, F16>(v + (int64_t)k0 * row_stride + kv * D, row_stride, nval, vts, tid);
    stage_k_rows<D, SPLIT, F16>(k + (int64_t)k0 * row_stride + kv * D, row_stride, nval, kt, tid);
    __syncthreads();
    store_vt_rows<D>(vts, vt, tid);
    if (app.rope_dim > 0 && kv == 0) {
        float2* tab = const_cast<float2*>(rope_table<D, SPLIT>(tiles, Hkv, n_tiles));
        constexpr int RPP = 256 / (D / 2);  // positions per pass
        const int j = tid % (D / 2);
        const bool rot = 2 * j < app.rope_dim;
        const double turns = rot ? rope_turns_per_pos(j, app.rope_dim, app.base) : 0.0;
        for (int r = tid / (D / 2); r < nval; r += RPP) {
            const int pos = lt * kBN + r;
            float c = 1.0f, sn = 0.0f;
            if (rot) rope_cos_sin(pos, turns, c, sn);
            tab[(int64_t)pos * (D / 2) + j] = float2{c, sn};
        }
    }
}

// ---------------------------------------------------------------------------
// An 8-bit store -> tiles (needle-core v3/model.rs: the int8 K/V store of a
// quantised session, each row its codes and one scale).  V is dequantised (code x
// its row's scale, rounded to bf16) into the V tiles above.  K: with I8 the codes
// stay int8, 64 rows x D bytes with the 16-byte chunks of a row swizzled as the
// V^T rows are (the operand of v_mfma_i32_32x32x32_i8); otherwise they are
// converted unchanged into the bf16 K tiles above (exact in bf16).  The tile's 64
// key scales (0 past the end of the sequence) go to ks_ws[(kv head, tile)][64]:
// the attention kernel multiplies the integer scores by them.
template <int D, bool I8>
__global__ __launch_bounds__(256) void stage_kv_q8_kernel(Q8Store q8, unsigned char* __restrict__ wsb,
                                                          float* __restrict__ ks_ws,
                                                          AttnSched sched, int Hkv) {
    constexpr int NCH = D / 8;
    constexpr int KT = I8 ? kBN * D : kBN * D * 2;  // K tile bytes
    __shared__ __attribute__((aligned(16))) __bf16 vts[D * kVts];
    const int tid = threadIdx.x;
    const int kv = blockIdx.x % Hkv;
    const int gt = blockIdx.x / Hkv;
    const int n_tiles = sched.n_tiles;
    const int s = find_seq(sched.tile_off, sched.n_seqs, gt);
    const int k0 = sched.koff[s] + (gt - sched.tile_off[s]) * kBN;  // the tile's key rows
    const int nval = min(kBN, sched.koff[s + 1] - k0);
    const int64_t row_stride = (int64_t)Hkv * D;
    unsigned char* ktb = wsb + ((int64_t)kv * n_tiles + gt) * KT;
    __bf16* vt = reinterpret_cast<__bf16*>(wsb + (int64_t)Hkv * n_tiles * KT) +
                 ((int64_t)kv * n_tiles + gt) * (kBN * D);
    const int8_t* kin = q8.k + (int64_t)k0 * row_stride + kv * D;
    const int8_t* vin = q8.v + (int64_t)k0 * row_stride + kv * D;
    if (tid < kBN)
        ks_ws[((int64_t)kv * n_tiles + gt) * kBN + tid] =
            tid < nval ? q8.ks[(int64_t)(k0 + tid) * Hkv + kv] : 0.0f;
    // V: 4 keys x 4 dims per block (4-byte code loads), dequantised, written to LDS as
    // four 4-key runs of V^T.  Block b: dims 4 (b % (D/4)) .., keys 4 (b / (D/4)) ..
    constexpr int VB = kBN * D / 16;
#pragma unroll
    for (int i = 0; i < VB / 256; ++i) {
        const int b = tid + 256 * i;
        const int d0 = 4 * (b % (D / 4)), key0 = 4 * (b / (D / 4));
        float r[4][4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool ok = key0 + e < nval;
            const uint32_t w = ok ? *reinterpret_cast<const uint32_t*>(vin + (key0 + e) * row_stride + d0) : 0u;
            const float sc = ok ? q8.vs[(int64_t)(k0 + key0 + e) * Hkv + kv] : 0.0f;
#pragma unroll
            for (int c = 0; c < 4; ++c) r[e][c] = (float)(int8_t)(w >> (8 * c)) * sc;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            bf16x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (__bf16)r[e][c];
            *reinterpret_cast<bf16x4*>(vts + (d0 + c) * kVts + key0) = x;
        }
    }
    if constexpr (I8) {
        // K: 16-byte chunks of codes, copied to their swizzled place
        constexpr int NC16 = D / 16;
        for (int i = tid; i < kBN * NC16; i += 256) {
            const int r = i / NC16, c = i % NC16;
            const uint4 w = r < nval ? *reinterpret_cast<const uint4*>(kin + r * row_stride + 16 * c)
                                     : uint4{0u, 0u, 0u, 0u};
            *reinterpret_cast<uint4*>(ktb + r * D + 16 * swz(r, c, NC16)) = w;
        }
    } else {
        // K: 8 codes (one 16-byte bf16 chunk) per step, to their swizzled place
        __bf16* kt = reinterpret_cast<__bf16*>(ktb);
        for (int i = tid; i < kBN * NCH; i += 256) {
            const int r = i / NCH, c = i % NCH;
            bf16x8 x;
            const uint2 w = r < nval ? *reinterpret_cast<const uint2*>(kin + r * row_stride + 8 * c)
                                     : uint2{0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                x[e] = (__bf16)(float)(int8_t)((e < 4 ? w.x : w.y) >> (8 * (e & 3)));
            *reinterpret_cast<bf16x8*>(kt + r * D + 8 * swz(r, c, NCH)) = x;
        }
    }
    __syncthreads();
    store_vt_rows<D>(vts, vt, tid);
}

// ---------------------------------------------------------------------------
template <int D, bool SPLIT, bool PREP, bool Q8, bool MERGE, bool F16>
__global__ __launch_bounds__(kThreads, 1) void attn_bf16_kernel(const float* __restrict__ q,
                                                                const __bf16* __restrict__ ws,
                                                                float* __restrict__ out,
                                                                AttnSched sched, AttnGeom geom,
                                                                PrepParams prep, Partials part,
                                                                Q8Store q8) {
    constexpr int KP = SPLIT ? 2 : 1;
    // Q8 with head_dim 128: int8 K tiles and v_mfma_i32_32x32x32_i8 scores
    constexpr bool I8 = Q8 && D == 128;
    constexpr int NCH = D / 8;            // 16-byte chunks per bf16 K row
    constexpr int KT = I8 ? kBN * D : KP * kBN * D * 2;  // K tile bytes
    constexpr int VT = kBN * D * 2;       // V tile bytes
    constexpr int NQS = D / 16;           // MFMA steps of K Q^T (bf16)
    constexpr int NQ8 = D / 32;           // MFMA steps of K Q^T (int8)
    constexpr int NCB = D / 32;           // 32-row blocks of O^T
    constexpr int QS = D + 4;             // f32 row stride of the epilogue staging
    constexpr int K_LOADS = KT / (kThreads * 16);  // 16-byte direct loads per thread
    constexpr int V_LOADS = VT / (kThreads * 16);
    static_assert(K_LOADS >= 1 && V_LOADS >= 1 && KT % (kThreads * 16) == 0 &&
                  VT % (kThreads * 16) == 0, "tiles are whole 8 KB workgroup loads");
    constexpr int SMEM_TILES = 2 * KT + 2 * VT;
    // Q8: a ring of four 64-float key-scale vectors after the tiles.  Slot t & 3 is
    // filled with K(t) and read by X(t) of both groups; it is refilled by K(t+4),
    // issued two phases after group B's X(t).
    constexpr int SMEM_RING = SMEM_TILES, RING_SLOT = kBN * 4;
    constexpr int SMEM_MAIN = SMEM_TILES + (Q8 ? 4 * RING_SLOT : 0);
    constexpr int SMEM_OUT = 4 * 32 * QS * 4;
    __shared__ __attribute__((aligned(16)))
    unsigned char smem[SMEM_MAIN > SMEM_OUT ? SMEM_MAIN : SMEM_OUT];

    const int tid = threadIdx.x;
    const int lane = tid & 63, hl = lane >> 5, ln = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool grp_b = wave >= 4;

    const WorkItem wi = decode_item(sched, geom, blockIdx.x);
    const int kv = wi.kv, s0 = wi.s0, s1 = wi.s1, q0 = wi.q0;
    // key rows of the sequence: [ks0, ks1); query row i sees keys <= i + dsh (over a
    // cached prefix its position is base + i - s0; plain prefill: ks0 = s0, dsh = 0)
    const int ks0 = wi.k0, ks1 = wi.k1, dsh = ks1 - s1;
    const int causal = geom.causal, H = geom.H, Hkv = geom.Hkv;
    const float qscale = geom.qscale;
    const int n_all = sched.n_tiles, tile0 = sched.tile_off[wi.sid];
    // key tiles of the item (with a sliding window it starts at its first row's first
    // visible key); with a key split this workgroup takes tiles [t_begin, t_begin + n_local)
    const KeyRange kr = item_key_range(sched, geom, wi, kBN);
    const int nt_seq = kr.nt_seq, t_begin = kr.t_begin, n_local = kr.t_end - kr.t_begin;
    const int win = causal ? geom.window : 0;
    if (n_local <= 0) return;  // (uniform: the whole workgroup leaves)
    const bool split = kr.n_chunks > 1;

    const int hloc = wave % geom.hpw, rblk = wave / geom.hpw;
    const int h = kv * geom.g + wi.chunk * geom.hpw + hloc;
    const int wq0 = q0 + rblk * 32;
    const bool active = wq0 < s1;
    const int wave_last =
        causal ? min((min(wq0 + 31, s1 - 1) + dsh - ks0) / kBN, nt_seq - 1) : nt_seq - 1;
    const int wave_first = win > 0 ? max(0, wq0 + dsh - win + 1 - ks0) / kBN : 0;
    // (with a window: the lowest key the wavefront's last row sees; below it, masks)
    const int wave_lo = wq0 + 31 + dsh - win + 1;
    const int qi = wq0 + ln;

    // ---- Q operand (B of K Q^T): for step s, lane (hl, ln) supplies
    // Q[qi][hl*D/2 + 8s + e], e = 0..7 -- the contraction order is free to permute.
    bf16x8 qop[NQS], qlo[SPLIT ? NQS : 1];
    // Q8: the row's scale x softmax scale x log2(e), kept out of the exact integer
    // scores and applied in the exponent (clamped above 0: a row of zero codes has
    // scores 0, and hidden keys stay -inf)
    float qf = 0.0f;
    intx4 qop8[I8 ? NQ8 : 1];
    if constexpr (I8) {
        // codes of Q[qi][hl*D/2 + 16s + j], j = 0..15, for int8 step s
        const bool ok = active && qi < s1;
        const int8_t* src = q8.q + ((int64_t)(ok ? qi : s0) * H + h) * D + hl * (D / 2);
#pragma unroll
        for (int s = 0; s < NQ8; ++s)
            qop8[s] = ok ? *reinterpret_cast<const intx4*>(src + 16 * s) : intx4{0, 0, 0, 0};
        qf = fmaxf((ok ? q8.qs[(int64_t)qi * H + h] : 0.0f) * qscale, 1e-30f);
    } else if constexpr (Q8) {
        // codes of Q[qi][hl*D/2 + 8s + e], exact in bf16
        const bool ok = active && qi < s1;
        const int8_t* src = q8.q + ((int64_t)(ok ? qi : s0) * H + h) * D + hl * (D / 2);
#pragma unroll
        for (int s = 0; s < NQS; s += 2) {
            const uint4 w = ok ? *reinterpret_cast<const uint4*>(src + 8 * s) : uint4{0, 0, 0, 0};
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 16; ++e)
                qop[s + e / 8][e % 8] = (__bf16)(float)(int8_t)(ww[e / 4] >> (8 * (e % 4)));
        }
        qf = fmaxf((ok ? q8.qs[(int64_t)qi * H + h] : 0.0f) * qscale, 1e-30f);
    } else {
        const bool ok = active && qi < s1;
        const float* src = q + ((int64_t)(ok ? qi : s0) * H + h) * D + hl * (D / 2);
        float xq[NQS][8];
#pragma unroll
        for (int s = 0; s < NQS; ++s) {
            floatx4 a = ok ? *reinterpret_cast<const floatx4*>(src + 8 * s) : floatx4{0, 0, 0, 0};
            floatx4 b = ok ? *reinterpret_cast<const floatx4*>(src + 8 * s + 4)
                           : floatx4{0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < 8; ++e) xq[s][e] = e < 4 ? a[e] : b[e - 4];
        }
        if constexpr (PREP) {
            // Fused entry: RMS-normalise and rotate the wavefront's 32 Q rows once.  The
            // two lanes of a row hold half of it each.
            const int n = prep.rope_dim, half = n >> 1;
            const float2* tab = rope_table<D, SPLIT>(ws, Hkv, n_all);
            float ss = 0.0f;
#pragma unroll
            for (int s = 0; s < NQS; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e) ss += xq[s][e] * xq[s][e];
            ss += other_half(ss);
            const float rs = 1.0f / sqrtf(ss * (1.0f / D) + prep.eps);
            // the norm weights of this lane half's dims, 16 bytes at a time (the pointer is
            // 16-byte aligned, as the entry points check)
            const floatx4* w4 = reinterpret_cast<const floatx4*>(prep.wq + hl * (D / 2));
#pragma unroll
            for (int s = 0; s < NQS; ++s) {
                const floatx4 wa = w4[2 * s], wb = w4[2 * s + 1];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    xq[s][e] = ok ? xq[s][e] * rs * (e < 4 ? wa[e] : wb[e - 4]) : 0.0f;
            }
            const int pos = ok ? qi + dsh - ks0 : 0;  // rows past the end: any valid table entry
            // table row of the position; two (cos, sin) pairs per 16-byte load (rows and
            // the table start on 16-byte boundaries)
            const float2* trow = tab + pos * (D / 2);
            auto pairs = [&](int j) {  // pairs j and j + 1 (j even)
                return *reinterpret_cast<const floatx4*>(trow + j);
            };
            if (n == D) {
                // dim c pairs with c +- D/2: the same register of the other lane half.
                // Registers are exchanged two at a time: swap(a, b) hands lanes 0-31
                // the upper half of a and lanes 32-63 the lower half of b, swap(b, a)
                // the other two, so each lane receives its partner of both.
#pragma unroll
                for (int s = 0; s < NQS; ++s)
#pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        const unsigned a = __builtin_bit_cast(unsigned, xq[s][e]);
                        const unsigned b = __builtin_bit_cast(unsigned, xq[s][e + 1]);
                        const auto ab = __builtin_amdgcn_permlane32_swap(a, b, false, false);
                        const auto ba = __builtin_amdgcn_permlane32_swap(b, a, false, false);
                        const float pa = __builtin_bit_cast(float, hl ? ba[0] : ab[1]);
                        const float pb = __builtin_bit_cast(float, hl ? ab[0] : ba[1]);
                        const float sg = hl ? 1.0f : -1.0f;
                        const floatx4 t = pairs(8 * s + e);
                        xq[s][e] = xq[s][e] * t[0] + sg * pa * t[1];
                        xq[s][e + 1] = xq[s][e + 1] * t[2] + sg * pb * t[3];
                    }
            } else if (n == D / 2) {
                // dims c < D/2 (lane half 0) pair with c + D/4: register step s + NQS/2
                if (hl == 0) {
#pragma unroll
                    for (int s = 0; s < NQS / 2; ++s)
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float a = xq[s][e], b = xq[s + NQS / 2][e];
                            const floatx4 t2 = pairs(8 * s + (e & ~1));
                            const float c = t2[2 * (e & 1)], sn = t2[2 * (e & 1) + 1];
                            xq[s][e] = a * c - b * sn;
                            xq[s + NQS / 2][e] = a * sn + b * c;
                        }
                }
            } else {
                // any other rope_dim: partners through LDS, four wavefronts at a time
                float* qs = reinterpret_cast<float*>(smem) + (wave & 3) * 32 * QS + ln * QS;
#pragma unroll
                for (int round = 0; round < 2; ++round) {
                    const bool mine = (wave >> 2) == round;
                    if (mine) {
#pragma unroll
                        for (int s = 0; s < NQS; ++s) {
                            *reinterpret_cast<floatx4*>(qs + hl * (D / 2) + 8 * s) =
                                floatx4{xq[s][0], xq[s][1], xq[s][2], xq[s][3]};
                            *reinterpret_cast<floatx4*>(qs + hl * (D / 2) + 8 * s + 4) =
                                floatx4{xq[s][4], xq[s][5], xq[s][6], xq[s][7]};
                        }
                    }
                    __syncthreads();
                    if (mine) {
#pragma unroll
                        for (int s = 0; s < NQS; ++s)
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                const int c = hl * (D / 2) + 8 * s + e;
                                if (c < n) {
                                    const int j = c < half ? c : c - half;
                                    const float yp = qs[c < half ? c + half : c - half];
                                    const float2 t = trow[j];
                                    xq[s][e] = c < half ? xq[s][e] * t.x - yp * t.y
                                                        : xq[s][e] * t.x + yp * t.y;
                                }
                            }
                    }
                    __syncthreads();
                }
            }
        }
#pragma unroll
        for (int s = 0; s < NQS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = xq[s][e] * qscale;
                qop[s][e] = to16<F16>(x);
                if constexpr (SPLIT) qlo[s][e] = (__bf16)(x - (float)qop[s][e]);
            }
    }
    // Q8: the key scales of this workgroup's tiles (64 per tile, after the V tiles)
    const float* ks_src =
        reinterpret_cast<const float*>(reinterpret_cast<const unsigned char*>(ws) +
                                       (int64_t)Hkv * n_all * (KT + VT)) +
        ((int64_t)kv * n_all + tile0 + t_begin) * kBN;

    // ---- tile sources in the workspace and per-lane LDS read addresses
    // (tile sources start at this workgroup's first tile; tiles are indexed locally)
    const unsigned char* kt_src = reinterpret_cast<const unsigned char*>(ws) +
                                  ((int64_t)kv * n_all + tile0 + t_begin) * KT;
    const unsigned char* vt_src = reinterpret_cast<const unsigned char*>(ws) +
                                  (int64_t)Hkv * n_all * KT +
                                  ((int64_t)kv * n_all + tile0 + t_begin) * VT;
    // K operand of step s, key block 0: row ln, chunk hl*NCH/2 + s (block 1: +32 rows)
    // (int8 tiles: row ln, 16-byte chunk hl*D/32 + s of the D-byte row, block 1: +32 rows)
    uint32_t kaddr[NQS];
#pragma unroll
    for (int s = 0; s < NQS; ++s)
        kaddr[s] = I8 ? (s < NQ8 ? ln * D + 16 * swz(ln, hl * (D / 32) + s, D / 16) : 0)
                      : ln * (D * 2) + 16 * swz(ln, hl * (NCH / 2) + s, NCH);
    // V^T operand of step s, row block 0: row ln, key group 2s + hl (block cb: +32cb rows)
    uint32_t vaddr[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) vaddr[s] = 2 * KT + ln * (kBN * 2) + 16 * swz(ln, 2 * s + hl, 8);

    // Direct-to-LDS copies: lane l of wavefront w moves bytes 16 (64 w + l) + 8192 i.
    // load_tiles(t): K of local tile t+1 and V of local tile t (those that exist).
    auto load_tiles = [&](int t) {
        if (t + 1 < n_local) {
            const unsigned char* src = kt_src + (int64_t)(t + 1) * KT + 16 * tid;
            unsigned char* dst = smem + ((t + 1) & 1) * KT + 1024 * wave;
#pragma unroll
            for (int i = 0; i < K_LOADS; ++i)
                __builtin_amdgcn_global_load_lds(src + 8192 * i, dst + 8192 * i, 16, 0, 0);
            // Q8: its 64 key scales into ring slot (t+1) & 3, four bytes a lane of wavefront 0
            if (Q8 && wave == 0)
                __builtin_amdgcn_global_load_lds(
                    reinterpret_cast<const unsigned char*>(ks_src + (int64_t)(t + 1) * kBN + lane),
                    smem + SMEM_RING + ((t + 1) & 3) * RING_SLOT, 4, 0, 0);
        }
        if (t >= 0 && t < n_local) {
            const unsigned char* src = vt_src + (int64_t)t * VT + 16 * tid;
            unsigned char* dst = smem + 2 * KT + (t & 1) * VT + 1024 * wave;
#pragma unroll
            for (int i = 0; i < V_LOADS; ++i)
                __builtin_amdgcn_global_load_lds(src + 8192 * i, dst + 8192 * i, 16, 0, 0);
        }
    };
    auto wait_loads = [] { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
    // Phase barrier: LDS reads done, then s_barrier.  Unlike __syncthreads() it
    // does not wait for the direct-to-LDS loads in flight (vmcnt); those are
    // waited for explicitly, one phase later.
    auto phase_barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

    floatx16 oacc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] = 0.0f;
    floatx16 sacc[2];
    intx16 sacc8[I8 ? 2 : 1];   // int8 scores (I8), converted in the X phase
    bf16x8 pop[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) pop[i][e] = (__bf16)0.0f;
    float m_run = -INFINITY;
    double l_run = 0.0;

    // M(t): P(t-1) V(t-1) into O, then S(t) = K(t) Q^T, as one stream of MFMAs
    // whose LDS operands are read kAhead reads ahead.  It always runs whole: P is
    // zero when there is nothing to add (before the first tile and past the
    // wavefront's last one, whose stale K reads are discarded), and the V buffer
    // read before the first tile is zeroed in the prologue.  PAR = t & 1.
    auto m_phase = [&](auto par_) {
        constexpr int PAR = decltype(par_)::value;
        constexpr int NPV = 4 * NCB;        // P.V: step s = i / NCB, block cb = i % NCB
        constexpr int NQK = I8 ? 2 * NQ8 : 2 * NQS * KP;  // K.Q^T: step s, key block kb, part
        constexpr int N = NPV + NQK;
        constexpr int kAhead = 4;
        const unsigned char* vb = smem + (PAR ^ 1) * VT;  // vaddr holds the V region offset
        const unsigned char* kb_ = smem + PAR * KT;
        auto rd = [&](int i) -> bf16x8 {
            if (i < NPV)
                return *reinterpret_cast<const bf16x8*>(vb + vaddr[i / NCB] +
                                                        (i % NCB) * 32 * kBN * 2);
            const int j = i - NPV;
            if constexpr (I8)  // 16 codes of key row ln (+32 kb), chunk of step j / 2
                return *reinterpret_cast<const bf16x8*>(kb_ + kaddr[j / 2] + (j % 2) * 32 * D);
            const int part = j % KP, kb = (j / KP) % 2, s = j / (2 * KP);
            return *reinterpret_cast<const bf16x8*>(kb_ + kaddr[s] + kb * 32 * D * 2 +
                                                    part * kBN * D * 2);
        };
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if constexpr (I8) sacc8[kb][r] = 0;
                else sacc[kb][r] = 0.0f;
            }
        bf16x8 opnd[N];
#pragma unroll
        for (int i = 0; i < kAhead; ++i) opnd[i] = rd(i);
#pragma unroll
        for (int i = 0; i < N; ++i) {
            if (i + kAhead < N) opnd[i + kAhead] = rd(i + kAhead);
            if (i < NPV) {
                // step s contracts keys 16s + 8(e/4) + 4hl + e%4: P registers 8(s%2)+e
                // of score block s/2, V^T key group 2s + hl
                oacc[i % NCB] = mfma16<F16>(opnd[i], pop[i / NCB], oacc[i % NCB]);
            } else {
                const int j = i - NPV;
                const int part = j % KP, kb = (j / KP) % 2, s = j / (2 * KP);
                if constexpr (I8) {
                    sacc8[j % 2] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                        __builtin_bit_cast(intx4, opnd[i]), qop8[j / 2], sacc8[j % 2], 0, 0, 0);
                } else if constexpr (SPLIT) {
                    // per key block: the two small cross terms first, then the high product
                    if (part == 1) {
                        sacc[kb] = mfma16<F16>(opnd[i], qop[s], sacc[kb]);
                        sacc[kb] = mfma16<F16>(opnd[i - 1], qlo[s], sacc[kb]);
                        sacc[kb] = mfma16<F16>(opnd[i - 1], qop[s], sacc[kb]);
                    }
                } else {
                    sacc[kb] = mfma16<F16>(opnd[i], qop[s], sacc[kb]);
                }
            }
        }
        // issue order: kAhead reads, then each MFMA followed by the next read
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int nm = (i < NPV || !SPLIT) ? 1 : ((i - NPV) % KP == 1 ? 3 : 0);
            if (nm == 1) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (nm == 3) __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
            if (i + kAhead < N) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // X(lt): scores of local tile lt -> P (bf16, B-operand layout), running max and sum.
    auto x_phase = [&](int lt) {
        const int t = t_begin + lt;
        if (lt < 0 || lt >= n_local || t > wave_last || t < wave_first) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 8; ++e) pop[i][e] = (__bf16)0.0f;
            return;
        }
        const int k0 = ks0 + t * kBN;
        if constexpr (Q8) {
            // integer scores x the scales of their key rows (register r of block kb:
            // key 32kb + 8(r/4) + 4hl + r%4 of the tile)
            const float* ksr =
                reinterpret_cast<const float*>(smem + SMEM_RING + (lt & 3) * RING_SLOT);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const floatx4 k4 =
                        *reinterpret_cast<const floatx4*>(ksr + 32 * kb + 8 * g + 4 * hl);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if constexpr (I8) sacc[kb][4 * g + i] = (float)sacc8[kb][4 * g + i] * k4[i];
                        else sacc[kb][4 * g + i] *= k4[i];
                    }
                }
        }
        // register r of block kb: key k0 + 32kb + 8(r/4) + 4hl + r%4.  A key is
        // hidden when it lies past min(qi + dsh, ks1-1) (causal) or past ks1-1, or
        // below the row's window.
        if ((causal && k0 + kBN - 1 > wq0 + dsh) || k0 + kBN > ks1 ||
            (win > 0 && k0 < wave_lo)) {
            const int lim = (causal ? min(qi + dsh, ks1 - 1) : ks1 - 1) - (k0 + 4 * hl);
            // (window: keys below the row's first visible one, qi + dsh - win + 1)
            const int lo = win > 0 ? qi + dsh - win + 1 - (k0 + 4 * hl) : -kBN;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int idx = 32 * kb + 8 * (r >> 2) + (r & 3);
                    if (idx > lim || idx < lo) sacc[kb][r] = -INFINITY;
                }
        }
        // Weights against the running max straight away; the lane's score max is
        // checked beside them.  Only when some score lies more than kLazyMax above
        // the running max (the first tile, or a real jump) is the row max taken and
        // the weights recomputed, so the result is that of taking the row max
        // first: m moves to it when it passes m + kLazyMax.
        // A row that has seen no key yet keeps m = -inf (over a cached prefix a row
        // can see no key of a tile, or of a split key range); exponents against
        // -1e30 then give 0 for its hidden keys, not NaN.
        // (Q8: scores are sacc x qf, qf > 0, so their max is max(sacc) x qf)
        const float lmax = fmaxf(max16(sacc[0]), max16(sacc[1])) * (Q8 ? qf : 1.0f);
        const float m_sub = fmaxf(m_run, -1e30f);
        // exponent of a weight: score - m
        auto ex = [&](float x, float m) { return Q8 ? fmaf(x, qf, -m) : x - m; };
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const bf16x2 pr = to16x2<F16>(__builtin_amdgcn_exp2f(ex(sacc[kb][r], m_sub)),
                                              __builtin_amdgcn_exp2f(ex(sacc[kb][r + 1], m_sub)));
                pop[2 * kb + (r >> 3)][r & 7] = pr[0];
                pop[2 * kb + (r >> 3)][(r & 7) + 1] = pr[1];
            }
        // (issued ahead of the check, not sunk below it onto the max's critical path)
        asm volatile("" : "+v"(pop[0]), "+v"(pop[1]), "+v"(pop[2]), "+v"(pop[3]));
        if (__any(lmax > m_run + kLazyMax)) {
            // (mt = -inf only in a row that sees no key here: no bump, weights 0)
            const float mt = max_halves(lmax);
            const bool bump = mt > m_run + kLazyMax;
            float alpha = bump ? __builtin_amdgcn_exp2f(m_run - mt) : 1.0f;
            if (bump) m_run = mt;
            const float m_new = fmaxf(m_run, -1e30f);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const bf16x2 pr =
                        to16x2<F16>(__builtin_amdgcn_exp2f(ex(sacc[kb][r], m_new)),
                                    __builtin_amdgcn_exp2f(ex(sacc[kb][r + 1], m_new)));
                    pop[2 * kb + (r >> 3)][r & 7] = pr[0];
                    pop[2 * kb + (r >> 3)][(r & 7) + 1] = pr[1];
                }
            l_run *= (double)alpha;
            // alpha is 1 in rows without a bump; hidden from the optimiser, which
            // would otherwise make the multiplication unconditional
            asm volatile("" : "+v"(alpha));
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
        }
        // the denominator sums the weights as rounded for the P.V product, so the
        // output is a weighted mean of V with exactly the weights that were applied
        float ps[2] = {0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bf16x2 pr = {pop[i][2 * e], pop[i][2 * e + 1]};
                ps[e & 1] = add_pair<F16>(pr, ps[e & 1]);
            }
        l_run += (double)(ps[0] + ps[1]);
    };

    // ---- prologue: K(0) in LDS, V buffer 1 (read by M(0) with P = 0) zeroed;
    // group B runs one phase behind group A
    for (int i = tid; i < VT / 16; i += kThreads)
        *reinterpret_cast<floatx4*>(smem + 2 * KT + VT + 16 * i) = floatx4{0.f, 0.f, 0.f, 0.f};
    load_tiles(-1);
    wait_loads();
    phase_barrier();
    if (grp_b) {
        load_tiles(0);
        phase_barrier();
    }
    // ---- main loop: per tile two phases, a barrier after each.  Loads of K(t+1)
    // and V(t) are issued in global phase 2t (A: before M(t); B: before X(t-1),
    // i.e. B issues tile t+1's loads before its X(t)) and waited for at the end of
    // global phase 2t+1.
    for (int t0 = 0; t0 <= n_local; t0 += 2) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int t = t0 + u;  // local tile index
            if (t > n_local) break;
            if (!grp_b) load_tiles(t);
            if (u == 0) m_phase(std::integral_constant<int, 0>{});
            else m_phase(std::integral_constant<int, 1>{});
            if (grp_b) wait_loads();
            phase_barrier();
            if (grp_b) load_tiles(t + 1);
            x_phase(t);
            if (!grp_b) wait_loads();
            phase_barrier();
        }
    }
    if (!grp_b) phase_barrier();

    // ---- epilogue: 1/l, transpose through LDS (four wavefronts at a time), coalesced rows
    // to the output, or for a split item to this unit's partial-result slot
    const double l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = l_tot > 0.0 ? (float)(1.0 / l_tot) : 0.0f;
    const size_t slot = (size_t)blockIdx.x * kWaves + wave;
    if (split && hl == 0) {
        part.ml[slot * 32 + ln] = float2{m_run, (float)l_tot};
    }
#pragma unroll
    for (int round = 0; round < 2; ++round) {
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
                const floatx4 x = *reinterpret_cast<const floatx4*>(os + r * QS + 4 * c4);
                if (split) {
                    *reinterpret_cast<floatx4*>(part.o + (slot * 32 + r) * D + 4 * c4) = x;
                } else if (row < s1) {
                    floatx4 y = x;
                    if (geom.gate)
                        y *= gate_factors(geom.gate, geom.gate_per_head, row, H, h, D,
                                          4 * c4);
                    *reinterpret_cast<floatx4*>(out + ((int64_t)row * H + h) * D + 4 * c4) = y;
                }
            }
        }
        if (round == 0) __syncthreads();
    }
    if constexpr (MERGE) {
        // the item's last unit to arrive merges every key chunk's partial result
        __shared__ int last_flag;
        const size_t item_slot = ((size_t)wi.item * geom.chunks + wi.chunk) * Hkv + kv;
        if (split && arrive_last(part, item_slot, kr.n_chunks, &last_flag)) {
            const size_t kstride = (size_t)geom.chunks * Hkv * kWaves;
            const size_t slot0 =
                (((size_t)wi.item * sched.max_chunks * geom.chunks + wi.chunk) * Hkv + kv) *
                    kWaves + wave;
            if (active)
                merge_slot<D>(part, slot0, kstride, kr.n_chunks, out, wq0, s1, H, h, geom.gate,
                              geom.gate_per_head, lane);
            if (tid == 0) reset_counter(part, item_slot);
        }
    }
}

// The launches of one call for fixed template arguments: tiles appended (kept tiles)
// or the rotary table and the staging kernel, then the attention kernel.
template <int D, bool SPLIT, bool PREP, bool F16>
void launch_bf16_kernels(const float* q, const float* k, const float* v, float* out, __bf16* w,
                         const AttnSched& sched, const AttnGeom& geom, const PrepParams& p,
                         bool prep_k, const Partials& part, int n_items, hipStream_t stream,
                         const TileAppend* app) {
    const dim3 sgrid((unsigned)sched.n_tiles * geom.Hkv), sblock(256);
    const dim3 grid((unsigned)n_items * sched.max_chunks * geom.chunks * geom.Hkv),
        block(kThreads);
    if (app) {
        const dim3 agrid((unsigned)(app->cum[app->n_seqs] * geom.Hkv));
        if (app->cum[app->n_seqs] > 0)
            hipLaunchKernelGGL((append_tiles_kernel<D, SPLIT, F16>), agrid, sblock, 0, stream, k,
                               v, w, *app, geom.Hkv);
    } else {
        if (PREP) {
            const dim3 tgrid((unsigned)((sched.max_len + kTabRows - 1) / kTabRows));
            hipLaunchKernelGGL((rope_table_kernel<D, SPLIT>), tgrid, sblock, 0, stream, w,
                               geom.Hkv, sched.n_tiles, sched.max_len, p.rope_dim, p.base);
        }
        if (PREP && prep_k)
            hipLaunchKernelGGL((stage_kv_bf16_kernel<D, SPLIT, true, F16>), sgrid, sblock, 0,
                               stream, k, v, w, sched, geom.Hkv, p);
        else
            hipLaunchKernelGGL((stage_kv_bf16_kernel<D, SPLIT, false, F16>), sgrid, sblock, 0,
                               stream, k, v, w, sched, geom.Hkv, p);
    }
    if (part.cnt)  // in-place merge of split items
        hipLaunchKernelGGL((attn_bf16_kernel<D, SPLIT, PREP, false, true, F16>), grid, block, 0,
                           stream, q, w, out, sched, geom, p, part, Q8Store{});
    else
        hipLaunchKernelGGL((attn_bf16_kernel<D, SPLIT, PREP, false, false, F16>), grid, block, 0,
                           stream, q, w, out, sched, geom, p, part, Q8Store{});
}

template <int D, bool PREP>
void launch_bf16_mode(bool split_qk, bool f16, const float* q, const float* k, const float* v,
                      float* out, __bf16* w, const AttnSched& sched, const AttnGeom& geom,
                      const PrepParams& p, bool prep_k, const Partials& part, int n_items,
                      hipStream_t stream, const TileAppend* app) {
    if (f16)
        launch_bf16_kernels<D, false, PREP, true>(q, k, v, out, w, sched, geom, p, prep_k, part,
                                                  n_items, stream, app);
    else if (split_qk)
        launch_bf16_kernels<D, true, PREP, false>(q, k, v, out, w, sched, geom, p, prep_k, part,
                                                  n_items, stream, app);
    else
        launch_bf16_kernels<D, false, PREP, false>(q, k, v, out, w, sched, geom, p, prep_k, part,
                                                   n_items, stream, app);
}

}  // namespace

hipError_t launch_attn_bf16(const float* q, const float* k, const float* v, float* out, void* ws,
                            const AttnSched& sched, const AttnGeom& geom, int D, bool split_qk,
                            bool f16, const PrepParams* prep, bool prep_k, const Partials& part,
                            int n_items, hipStream_t stream, const TileAppend* app) {
    __bf16* w = static_cast<__bf16*>(ws);
    const PrepParams p = prep ? *prep : PrepParams{nullptr, nullptr, nullptr, 0, 0.0f, 0.0};
    if (D == 128) {
        if (prep) launch_bf16_mode<128, true>(split_qk, f16, q, k, v, out, w, sched, geom, p,
                                              prep_k, part, n_items, stream, app);
        else launch_bf16_mode<128, false>(split_qk, f16, q, k, v, out, w, sched, geom, p,
                                          prep_k, part, n_items, stream, app);
    } else {
        if (prep) launch_bf16_mode<64, true>(split_qk, f16, q, k, v, out, w, sched, geom, p,
                                             prep_k, part, n_items, stream, app);
        else launch_bf16_mode<64, false>(split_qk, f16, q, k, v, out, w, sched, geom, p,
                                         prep_k, part, n_items, stream, app);
    }
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && sched.max_chunks > 1 && !part.cnt)
        e = launch_attn_combine(part, out, sched, geom, D, kWaves, kBN, n_items, stream);
    return e;
}

hipError_t launch_attn_q8(const Q8Store& st8, float* out, void* ws, const AttnSched& sched,
                          const AttnGeom& geom, int D, const Partials& part, int n_items,
                          hipStream_t stream) {
    __bf16* w = static_cast<__bf16*>(ws);
    unsigned char* wb = static_cast<unsigned char*>(ws);
    // head_dim 128: int8 K tiles (64 x D bytes); 64: bf16 K tiles.  Then the bf16 V
    // tiles, then the key scales (the attention kernel finds them the same way).
    float* ks_ws = reinterpret_cast<float*>(wb + q8_tile_bytes(sched.n_tiles, geom.Hkv, D));
    const bool merge = part.cnt != nullptr;  // in-place merge of split items
    const PrepParams p{nullptr, nullptr, nullptr, 0, 0.0f, 0.0};
    const dim3 sgrid((unsigned)sched.n_tiles * geom.Hkv), sblock(256);
    const dim3 grid((unsigned)n_items * sched.max_chunks * geom.chunks * geom.Hkv),
        block(kThreads);
    if (D == 128) {
        hipLaunchKernelGGL((stage_kv_q8_kernel<128, true>), sgrid, sblock, 0, stream, st8, wb,
                           ks_ws, sched, geom.Hkv);
        if (merge)
            hipLaunchKernelGGL((attn_bf16_kernel<128, false, false, true, true, false>), grid, block, 0,
                               stream, nullptr, w, out, sched, geom, p, part, st8);
        else
            hipLaunchKernelGGL((attn_bf16_kernel<128, false, false, true, false, false>), grid, block, 0,
                               stream, nullptr, w, out, sched, geom, p, part, st8);
    } else {
        hipLaunchKernelGGL((stage_kv_q8_kernel<64, false>), sgrid, sblock, 0, stream, st8, wb,
                           ks_ws, sched, geom.Hkv);
        if (merge)
            hipLaunchKernelGGL((attn_bf16_kernel<64, false, false, true, true, false>), grid, block, 0,
                               stream, nullptr, w, out, sched, geom, p, part, st8);
        else
            hipLaunchKernelGGL((attn_bf16_kernel<64, false, false, true, false, false>), grid, block, 0,
                               stream, nullptr, w, out, sched, geom, p, part, st8);
    }
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && sched.max_chunks > 1 && !merge)
        e = launch_attn_combine(part, out, sched, geom, D, kWaves, kBN, n_items, stream);
    return e;
}

}  // namespace pfa
