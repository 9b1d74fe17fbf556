// pfa_device.h -- small device helpers shared by the libpfa kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pfa_internal.h"

namespace pfa {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr double kInvTwoPi = 0.15915494309189533577;  // 1 / (2 pi)

// A raw buffer resource over `bytes` bytes from `base` (wavefront-uniform).
// Buffer loads whose per-lane byte offset (the VGPR offset) falls outside
// [0, bytes) return zeros, so tiles that run past the end of a sequence need no
// branches.  0x00020000 is the gfx9 data-format word of an untyped buffer.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ floatx4 buffer_load_f4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// Sum over the 64 lanes of a wavefront (every lane receives the total).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// Online softmax with a lazy running max: the max used as the exponent offset moves
// only when a tile's score max passes it by more than this (log2 units), so weights
// stay below 2^8 and the output and denominator are rescaled only when it moves.
constexpr float kLazyMax = 8.0f;

// v_max3_f32 without the NaN-quieting operand canonicalisation fmaxf gets (the
// scores are MFMA results or -inf, never signalling NaNs)
__device__ __forceinline__ float max3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// max of the 16 registers of a score block
__device__ __forceinline__ float max16(const floatx16& x) {
    float m = max3(x[0], x[1], x[2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) m = max3(m, x[r], x[r + 1]);
    return max3(m, x[15], x[15]);
}

// The value lane l ^ 32 holds.  v_permlane32_swap(a, b) leaves lanes 0-31 of a in
// both halves of its first result and lanes 32-63 of b in both halves of its
// second.  The second operand goes through an empty asm so that the compiler
// cannot treat the two operands, and hence the two results, as one value (it
// folds the second result into the first when both operands are the same value).
__device__ __forceinline__ float other_half(float x) {
    unsigned a = __builtin_bit_cast(unsigned, x), b = a;
    asm volatile("" : "+v"(b));
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}

// max over the two lanes of one query (lanes l and l ^ 32)
__device__ __forceinline__ float max_halves(float x) { return fmaxf(x, other_half(x)); }

// Sum over the 64 lanes of a wavefront: DPP rotations and quad permutations
// inside each 16-lane row (plain VALU operand modifiers), then two cross-row
// exchanges.  Every lane receives the total.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                  CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_sum_dpp(float x) {
    x += dpp_f32<0x128>(x);  // row_ror:8
    x += dpp_f32<0x124>(x);  // row_ror:4
    x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}

// Max over the 64 lanes of a wavefront (every lane receives it).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

// Max over the 64 lanes with DPP inside each 16-lane row, then two cross-row exchanges
// (as wave_sum_dpp).  Every lane receives it.
__device__ __forceinline__ float wave_max_dpp(float x) {
    x = fmaxf(x, dpp_f32<0x128>(x));  // row_ror:8
    x = fmaxf(x, dpp_f32<0x124>(x));  // row_ror:4
    x = fmaxf(x, dpp_f32<0x4E>(x));   // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp_f32<0xB1>(x));   // quad_perm [1,0,3,2]
    x = fmaxf(x, __shfl_xor(x, 16, 64));
    x = fmaxf(x, __shfl_xor(x, 32, 64));
    return x;
}

// 8-bit quantisation of a (token, head) row (needle-core v3/model.rs, `quant_rows` /
// `quantize_rows`, whose bodies the page does not print).  This library's reading of
// the rule: the row's scale is its largest magnitude over 127, and a value's code is the
// nearest integer to value / scale (ties to even) within -127..127; a row of zeros has
// scale 0 and codes 0.  The divisor 127 and the tie direction are that reading's
// choices, not the page's.  IEEE single-precision division, so the codes are those of
// any correctly rounded implementation.
__device__ __forceinline__ float quant8_scale(float amax) { return amax / 127.0f; }
__device__ __forceinline__ int quant8(float x, float scale) {
    const float c = scale > 0.0f ? __builtin_rintf(x / scale) : 0.0f;
    return (int)fminf(fmaxf(c, -127.0f), 127.0f);
}

// Sum over groups of `width` consecutive lanes (width a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// Turns per position of rotary pair j: base^(-2j/n) / (2 pi), in f64.
__device__ __forceinline__ double rope_turns_per_pos(int j, int n, double base) {
    return pow(base, -2.0 * (double)j / (double)n) * kInvTwoPi;
}

// cos and sin of the rotary angle pos * base^(-2j/n).  The angle is formed in
// f64 as a number of turns and reduced to [-1/2, 1/2] turn there, so only the
// final sincos runs in f32 on an argument of at most pi: the result keeps f32
// accuracy at any position (an f32 angle would lose ~1e-3 rad near 16k).  No
// multiply-add contraction (here and in norm_rope_row): every kernel that inlines
// them rounds the same operations, so they agree bit for bit.
__device__ __forceinline__ void rope_cos_sin(int pos, double turns_per_pos, float& c, float& s) {
#pragma clang fp contract(off)
    double r = (double)pos * turns_per_pos;
    r -= rint(r);
    sincospif((float)(2.0 * r), &s, &c);
}

// Factors of a gated output for elements c .. c+3 of head h of output row `row`: the
// logistic sigmoid of the gate, one value per element (gate [rows, H*D]) or per head
// (gate [rows, H]).  1 / (1 + 2^(-g log2 e)): saturates to exactly 0 and 1.
__device__ __forceinline__ floatx4 gate_factors(const float* gate, int per_head, int64_t row,
                                                int H, int h, int D, int c) {
    floatx4 g;
    if (per_head) {
        const float x = gate[row * H + h];
        g = floatx4{x, x, x, x};
    } else {
        g = *reinterpret_cast<const floatx4*>(gate + (row * H + h) * D + c);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) g[e] = 1.0f / (1.0f + __builtin_amdgcn_exp2f(-g[e] * kLog2e));
    return g;
}

// Index of the packed sequence holding token t: the largest s < n_seqs with
// off[s] <= t (empty sequences resolve to the next non-empty one).
__device__ __forceinline__ int find_seq(const int* off, int n_seqs, int t) {
    int lo = 0, hi = n_seqs;
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (off[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
}

// One workgroup's share of the attention work (see AttnSched): K/V head, head
// chunk of the group, the sequence and query super-block it covers, and which
// chunk of that super-block's key tiles.
struct WorkItem {
    int kv, chunk, sb;   // K/V head, head chunk, super-block index in the sequence
    int kc;              // key chunk (0 when the key range is not split)
    int item;            // index in the longest-first item order
    int sid;             // sequence index
    int s0, s1;          // the sequence's query rows [s0, s1)
    int k0, k1;          // its key rows [k0, k1); query row i sees keys <= i + k1 - s1
    int q0;              // first query row of the super-block
};

// item -> sequence and super-block (segment decode of the longest-first order).
// Host and device: the library's plan report (pfa_attn_units) decodes the grid with
// the same code the kernels run.
template <class Sched>
__host__ __device__ __forceinline__ void decode_seq(const Sched& sched, WorkItem& w) {
    int seg = 0;
    while (w.item >= sched.seg_start[seg + 1]) ++seg;
    const int local = w.item - sched.seg_start[seg];
    const int per = seg + 1;
    const int sid = sched.order[local % per];
    w.sb = sched.seg_top[seg] - 1 - local / per;
    w.sid = sid;
    w.s0 = sched.off[sid];
    w.s1 = sched.off[sid + 1];
    w.k0 = sched.koff[sid];
    w.k1 = sched.koff[sid + 1];
    w.q0 = w.s0 + w.sb * sched.rows_per_item;
}

// blockIdx.x -> work unit.  The K/V head is the fastest-varying index (so the
// workgroups that the dispatcher deals to the 8 XCDs in turn share heads), then
// the head chunk, then the key chunk, and the longest-first item order slowest.
template <class Sched, class Geom>
__host__ __device__ __forceinline__ WorkItem decode_item(const Sched& sched, const Geom& geom, int bid) {
    WorkItem w;
    w.kv = bid % geom.Hkv;
    bid /= geom.Hkv;
    w.chunk = bid % geom.chunks;
    bid /= geom.chunks;
    w.kc = bid % sched.max_chunks;
    w.item = bid / sched.max_chunks;
    decode_seq(sched, w);
    return w;
}

// The key tiles (of tile_keys keys) a work unit visits.  Causal: an item's tiles run to
// its last query row's last visible key; with a sliding window they start at its first
// row's first visible key.  With a key split (sched.kchunk > 0) the item's tiles are cut
// into chunks of kchunk tiles and the unit takes chunk wi.kc: tiles [t_begin, t_end).
// A unit whose chunk lies past the item's tiles has t_begin >= t_end (it does nothing).
struct KeyRange {
    int nt_seq;    // tiles over the sequence's key rows
    int n_tiles;   // one past the item's last tile
    int t_first;   // the item's first tile
    int n_chunks;  // key chunks of the item (1: not split)
    int t_begin, t_end;
};
template <class Sched, class Geom>
__host__ __device__ __forceinline__ KeyRange item_key_range(const Sched& sched, const Geom& geom,
                                                            const WorkItem& wi, int tile_keys) {
    KeyRange r;
    const int dsh = wi.k1 - wi.s1;  // query row i sees keys <= i + dsh
    r.nt_seq = (wi.k1 - wi.k0 + tile_keys - 1) / tile_keys;
    const int last_row = (wi.q0 + sched.rows_per_item < wi.s1 ? wi.q0 + sched.rows_per_item
                                                               : wi.s1) - 1;
    r.n_tiles = geom.causal ? (last_row + dsh - wi.k0) / tile_keys + 1 : r.nt_seq;
    const int win = geom.causal ? geom.window : 0;
    const int lo = wi.q0 + dsh - win + 1 - wi.k0;
    r.t_first = win > 0 ? (lo > 0 ? lo : 0) / tile_keys : 0;
    const int kchunk = sched.kchunk > 0 ? sched.kchunk : r.n_tiles - r.t_first;
    r.n_chunks = (r.n_tiles - r.t_first + kchunk - 1) / kchunk;
    r.t_begin = r.t_first + wi.kc * kchunk;
    r.t_end = r.t_begin + kchunk < r.n_tiles ? r.t_begin + kchunk : r.n_tiles;
    return r;
}

// ---------------------------------------------------------------------------
// QK-norm + NeoX RoPE of one head row held by one wavefront, lane L holding dims L + 64 e
// (e < D / 64): the arithmetic of qknorm_rope_kernel, shared with the kernels that prepare
// K rows on their way into the bf16 tiles, so that both give the same bits.
//
// Rotary pair (j, j + n/2): with n == D == 128 both dims of a pair sit in the same lane;
// with n == 64 the partner is lane L ^ 32; any other even n takes a general shuffle.
enum PairMode { kPairInLane = 0, kPairXor32 = 1, kPairGeneral = 2 };

// Per-lane rotary constants: which pair each of the lane's dims belongs to.
template <int D>
struct RopeLane {
    double turns[D / 64];  // turns per position of the pair (0: not rotated)
    float sgn[D / 64];     // -1 for the first dim of a pair, +1 for the second
    int src[D / 64], slot[D / 64];  // the partner dim's lane and register
    bool rot[D / 64];
};
template <int D>
__device__ __forceinline__ RopeLane<D> rope_lane(int lane, int n, double base) {
    RopeLane<D> L;
    const int half = n >> 1;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) {
        const int c = lane + 64 * e;
        L.rot[e] = c < n;
        const bool first = c < half;
        const int j = first ? c : c - half;
        const int p = first ? c + half : c - half;
        L.sgn[e] = first ? -1.0f : 1.0f;
        L.src[e] = p & 63;
        L.slot[e] = p >> 6;
        L.turns[e] = L.rot[e] ? rope_turns_per_pos(j, n, base) : 0.0;
    }
    return L;
}
// cos / sin of the lane's dims at position pos.
template <int D>
__device__ __forceinline__ void rope_lane_angles(const RopeLane<D>& L, int pos, float* cs,
                                                 float* sn) {
#pragma unroll
    for (int e = 0; e < D / 64; ++e) {
        if (L.rot[e]) {
            rope_cos_sin(pos, L.turns[e], cs[e], sn[e]);
        } else {
            cs[e] = 1.0f;
            sn[e] = 0.0f;
        }
    }
}
// o = RoPE(x * w / rms(x)) of one row (x, o: the lane's dims; wv: the lane's weights).
template <int D, int MODE>
__device__ __forceinline__ void norm_rope_row(const float* x, const float* wv, const float* cs,
                                              const float* sn, const RopeLane<D>& L, float eps,
                                              float* o) {
#pragma clang fp contract(off)
    constexpr int E = D / 64;
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) ss += x[e] * x[e];
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss * (1.0f / D) + eps);
    float y[E];
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] = x[e] * r * wv[e];
    if (MODE == kPairInLane) {
        // n == D == 128: dims L and L + 64 are the two halves of pair L.
        o[0] = y[0] * cs[0] - y[E - 1] * sn[0];
        o[E - 1] = y[E - 1] * cs[0] + y[0] * sn[0];
    } else if (MODE == kPairXor32) {
        // n == 64: the partner of dim L (< 64) is dim L ^ 32, in lane L ^ 32.
        const float pv = __shfl_xor(y[0], 32, 64);
        o[0] = y[0] * cs[0] + L.sgn[0] * pv * sn[0];
#pragma unroll
        for (int e = 1; e < E; ++e) o[e] = y[e];
    } else {
        float pv[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float best = 0.0f;
#pragma unroll
            for (int sl = 0; sl < E; ++sl) {
                const float cand = __shfl(y[sl], L.src[e], 64);
                if (L.slot[e] == sl) best = cand;
            }
            pv[e] = best;
        }
#pragma unroll
        for (int e = 0; e < E; ++e)
            o[e] = L.rot[e] ? y[e] * cs[e] + L.sgn[e] * pv[e] * sn[e] : y[e];
    }
}

// ---------------------------------------------------------------------------
// In-place merge of a split item's partial results (see Partials).
//
// Units of one item may run on different XCDs, each with its own L2, so the hand-over
// follows the agent-scope memory model: every wavefront's partial-result stores complete
// (s_waitcnt vmcnt(0), then a workgroup barrier), one thread releases them at agent scope
// (an L2 write-back) before counting the unit's arrival, and the last unit to arrive
// acquires at agent scope (an L1 / L2 invalidate) before it reads the other units'
// results with ordinary loads.

// Called by every thread of a workgroup once each of its wavefronts has issued the
// stores of its partial result: counts the unit's arrival on counter `c` and returns,
// in every thread, whether this unit is the item's last (n_chunks arrivals).  `flag` is
// one int of LDS.  The compare-and-swap retries only while other units change the
// counter (at most n_chunks - 1 times); it never waits for anything.
__device__ __forceinline__ bool arrive_last(const Partials& part, size_t c, int n_chunks,
                                            int* flag) {
    __builtin_amdgcn_s_waitcnt(0);  // this wavefront's partial-result stores have completed
    __syncthreads();                // ... and every other wavefront's
    if (threadIdx.x == 0) {
        // release: the unit's partial results are visible at agent scope before its arrival
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        unsigned long long* p = part.cnt + c;
        unsigned long long old = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        unsigned long long nw;
        do {
            nw = (old >> 16) == part.tag ? old + 1 : (part.tag << 16) | 1ull;
        } while (!__hip_atomic_compare_exchange_strong(p, &old, nw, __ATOMIC_RELAXED,
                                                       __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT));
        const bool last = (int)(nw & 0xFFFF) == n_chunks;
        // acquire: the last unit sees every other unit's released results
        if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        *flag = last ? 1 : 0;
    }
    __syncthreads();
    return *flag != 0;
}

// The last unit leaves the counter 0 (after its merge has read everything).
__device__ __forceinline__ void reset_counter(const Partials& part, size_t c) {
    __hip_atomic_store(part.cnt + c, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge of one wavefront slot's key chunks (32 query rows of head h, rows row0 .. row0 +
// 31, those below s1 real; 2 <= n_chunks <= kMergeChunks) into `out`.  The softmax over
// the union of the chunks' keys, with M = max_k m_k and w_k = l_k 2^(m_k - M) (m in log2
// units, as the attention kernels keep it), is O = sum_k w_k (O_k / l_k) / sum_k w_k --
// the rescaling the online softmax applies between tiles; a chunk that saw none of a
// row's keys has l_k = 0 and weight 0.  Chunk k sits in slot slot0 + k * kstride.
// Lane L (< 32) forms the weights of row L; the rows themselves are read coalesced,
// load instruction i of a chunk taking float4 number 64 i + L of the slot (row
// (64 i + L) / (D / 4)), whose weight comes from the row's lane by a shuffle.  Every
// chunk's (m, l) and the first two chunks' rows are loaded together, then two chunks'
// rows per round trip.  An optional gate multiplies the merged rows (out = O *
// sigmoid(gate)).
template <int D>
__device__ __forceinline__ void merge_slot(const Partials& part, size_t slot0, size_t kstride,
                                           int n_chunks, float* out, int row0, int s1, int H,
                                           int h, const float* gate, int gate_per_head,
                                           int lane) {
    constexpr int F4 = D / 4;          // float4 per row
    constexpr int NV = 32 * F4 / 64;   // float4 per lane and chunk
    constexpr int RPI = 64 / F4;       // rows per load instruction
    const int r = lane & 31;
    auto load_rows = [&](int k, floatx4* x) {
        const floatx4* src =
            reinterpret_cast<const floatx4*>(part.o + (slot0 + (size_t)k * kstride) * 32 * D);
#pragma unroll
        for (int i = 0; i < NV; ++i) x[i] = src[64 * i + lane];
    };
    float m[kMergeChunks], l[kMergeChunks];
#pragma unroll
    for (int k = 0; k < kMergeChunks; ++k) {
        m[k] = -INFINITY;
        l[k] = 0.0f;
        if (k < n_chunks) {
            const float2 ml = part.ml[(slot0 + (size_t)k * kstride) * 32 + r];
            m[k] = ml.x;
            l[k] = ml.y;
        }
    }
    floatx4 xa[NV], xb[NV];
    load_rows(0, xa);
    load_rows(1, xb);
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < kMergeChunks; ++k)
        if (l[k] > 0.0f) mx = fmaxf(mx, m[k]);
    float w[kMergeChunks], den = 0.0f;
#pragma unroll
    for (int k = 0; k < kMergeChunks; ++k) {
        w[k] = l[k] > 0.0f ? l[k] * __builtin_amdgcn_exp2f(m[k] - mx) : 0.0f;
        den += w[k];
    }
    // weight of chunk k for the row of this lane's i-th float4
    auto wrow = [&](float wk, int i) { return __shfl(wk, RPI * i + lane / F4, 64); };
    floatx4 acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = wrow(w[0], i) * xa[i] + wrow(w[1], i) * xb[i];
#pragma unroll
    for (int k = 2; k < kMergeChunks; k += 2) {
        if (k < n_chunks) {  // (uniform)
            load_rows(k, xa);
            load_rows(k + 1 < n_chunks ? k + 1 : k, xb);
            const float wb = k + 1 < n_chunks ? w[k + 1] : 0.0f;
#pragma unroll
            for (int i = 0; i < NV; ++i) acc[i] += wrow(w[k], i) * xa[i] + wrow(wb, i) * xb[i];
        }
    }
    const float inv_r = den > 0.0f ? 1.0f / den : 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int rr = RPI * i + lane / F4, c4 = lane % F4;
        const int row = row0 + rr;
        const float inv = __shfl(inv_r, rr, 64);
        if (row < s1) {
            floatx4 y = acc[i] * inv;
            if (gate) y *= gate_factors(gate, gate_per_head, row, H, h, D, 4 * c4);
            *reinterpret_cast<floatx4*>(out + ((int64_t)row * H + h) * D + 4 * c4) = y;
        }
    }
}

}  // namespace pfa
