// pfa_internal.h -- types shared by the host entry points and the kernels of
// libpfa.  Not part of the public ABI (that is include/pfa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pfa.h"

namespace pfa {

// Packed-sequence boundaries, passed to kernels by value (kernel arguments),
// so no device buffer and no host-to-device copy is needed.  Sequence s owns
// rows off[s] .. off[s+1]-1 of the query-side tensors and rows koff[s] ..
// koff[s+1]-1 of the key/value side, at least as many: its first
// base_s = (koff[s+1] - koff[s]) - (off[s+1] - off[s]) key rows are a cached
// prefix, and its query rows sit at positions base_s, base_s + 1, ... (plain
// prefill: koff = off, base 0).
struct SeqTable {
    int n_seqs;
    int off[PFA_MAX_SEQS + 1];   // cumulative query-row offsets, off[n_seqs] = T
    int koff[PFA_MAX_SEQS + 1];  // cumulative key-row offsets
};

// Work schedule of the attention kernels, also passed by value.
//
// A work item is one (sequence, query super-block) pair; a super-block is
// rows_per_item consecutive query rows of one sequence.  Items are ordered
// longest first: the causal cost of super-block b is about b + 1 key tiles, so
// listing super-blocks from the top index down, across all sequences at once,
// is longest-processing-time-first order.  With the sequences sorted by their
// super-block count (order[]), the k+1 longest sequences are exactly the ones
// that have a super-block at levels seg_top[k+1] < level <= seg_top[k]; segment
// k holds those levels, k+1 items per level.
struct AttnSched {
    int n_seqs;
    int n_segs;                      // segments in use
    int rows_per_item;               // query rows per super-block (32 * row blocks)
    int off[PFA_MAX_SEQS + 1];       // as SeqTable::off
    int koff[PFA_MAX_SEQS + 1];      // as SeqTable::koff
    int seg_start[PFA_MAX_SEQS + 1]; // first item of each segment; [n_segs] = item count
    int seg_top[PFA_MAX_SEQS];       // super-block count of the (k+1)-th longest sequence
    int32_t order[PFA_MAX_SEQS];     // sequence ids, most super-blocks first (32-bit: scalar loads)
    // 64-key tiles of the bf16 workspace (see launch_attn_bf16): sequence s owns
    // tiles tile_off[s] .. tile_off[s+1]-1 of each K/V head (its key rows); n_tiles
    // in all.
    int n_tiles;
    int tile_off[PFA_MAX_SEQS + 1];
    int max_len;                     // most key rows of a sequence (rotary table rows)
    // Key split for short inputs: when the items alone cannot fill the GPU, each
    // item's key tiles are cut into chunks of kchunk tiles, one workgroup each
    // (grid = items x max_chunks x head chunks x K/V heads; chunk slots past an
    // item's count exit at once).  Items with more than one chunk write partial
    // results, merged in place by the item's last unit (max_chunks <= kMergeChunks)
    // or by attn_combine_kernel (see Partials).  kchunk = 0: no split (max_chunks 1).
    int kchunk;
    int max_chunks;
    // f32 kernel without a key split: workgroup j takes item j, then item
    // n_items - 1 - j (n_items = seg_start[n_segs]); the grid has (n_items + 1) / 2
    // item slots.  0: one item per workgroup.
    int paired;
};

// Partial results of a split item, per work unit (blockIdx) and wavefront:
// 32 rows x D of O / l (f32), and per row (m, l): running max (log2 units) and
// softmax denominator.  An empty wavefront writes m = -inf, l = 0.
//
// Two ways to merge them.  When every item has at most kMergeChunks chunks, in place:
// each unit counts its arrival on its item's counter once its partial result is
// stored, and the unit that arrives last merges all of them into the output (no
// second launch; the counters are `cnt`).  A counter is [tag : 48 bits | arrivals :
// 16 bits]; a value whose tag is not this call's counts as no arrivals, so the
// workspace needs no clearing, and the merging unit leaves it 0 (a replayed graph,
// whose tag is fixed, finds it so).  Otherwise (cnt null) attn_combine_kernel merges
// them in a second launch, which spreads the many chunks of a long cache over more
// workgroups.
constexpr int kMergeChunks = 4;
struct Partials {
    float* o;                  // [units][waves][32][D]
    float2* ml;                // [units][waves][32]
    unsigned long long* cnt;   // [items][head chunks][Hkv] arrival counters, or null
    unsigned long long tag;    // this call's tag, 1 .. 2^48 - 1 (in-place merge only)
};
// Bytes of the partial results and, for the in-place merge, `counters` counters
// (after the results, 256-byte aligned).
inline size_t partials_bytes(int units, int waves, int D, long long counters) {
    const size_t b = (size_t)units * waves * 32 * (D * 4 + 8);
    return counters ? ((b + 255) & ~(size_t)255) + (size_t)counters * 8 : b;
}
// The parts of a partial-result region at `base` (cnt null without counters).
inline Partials partials_at(void* base, int units, int waves, int D, long long counters,
                            unsigned long long tag) {
    char* w = static_cast<char*>(base);
    const size_t ob = (size_t)units * waves * 32 * D * 4, mb = (size_t)units * waves * 32 * 8;
    return Partials{reinterpret_cast<float*>(w), reinterpret_cast<float2*>(w + ob),
                    counters ? reinterpret_cast<unsigned long long*>(
                                   w + ((ob + mb + 255) & ~(size_t)255))
                             : nullptr,
                    tag};
}

// Geometry common to the attention launches.
struct AttnGeom {
    int H, Hkv, g;          // query heads, K/V heads, group size
    int hpw;                // query heads per workgroup (one wave each per row block)
    int rb;                 // 32-row blocks per workgroup
    int chunks;             // workgroups per K/V head per item (g / hpw)
    float qscale;           // softmax scale * log2(e), folded into Q
    int causal;
    int window;             // causal only: keys a row sees, its own included (0: all)
    // gated output: out = O * sigmoid(gate), gate [T_q, H*D] per element or [T_q, H] per
    // head (gate_per_head); applied where the final output rows are stored
    const float* gate;      // null: no gate
    int gate_per_head;
};

// Rotary + norm parameters for the fused entry.
struct PrepParams {
    const float* wq;
    const float* wk;
    float* k_rot_out;       // may be null
    int rope_dim;
    float eps;
    double base;            // rotary frequency base
};

// An 8-bit store (needle-core v3/model.rs, the int8 K/V store of a quantised session):
// int8 codes [rows, heads * D] and one f32 scale per (row, head), [rows, heads]; a value
// is its code times its row's scale.  Q, K and V each have one.
struct Q8Store {
    const int8_t* q;
    const float* qs;
    const int8_t* k;
    const float* ks;
    const int8_t* v;
    const float* vs;
};
// Outputs of the QK-norm + RoPE pass of a quantised session: Q codes per query row, K
// and V codes per key row (as k_out / v_out of launch_qknorm_rope); null parts skipped.
struct Q8Rows {
    int8_t* q;
    float* qs;
    int8_t* k;
    float* ks;
    int8_t* v;
    float* vs;
};

// Launchers (defined next to their kernels).  They only enqueue.
// QK-norm + RoPE of T query-side rows (H = 0: K rows only).  K rows go to
// k_out at the key rows the sequence table gives (the same rows for plain
// prefill); with v_out, the V rows are copied there too.
hipError_t launch_qknorm_rope(const float* q_in, const float* k_in, float* q_out, float* k_out,
                              const float* v_in, float* v_out, const float* wq, const float* wk,
                              const SeqTable& seqs, int T, int H, int Hkv, int D, int rope_dim,
                              float base, float eps, hipStream_t stream);

// The same pass for a quantised session: Q and K normalised and rotated, then Q, K and V
// quantised per (token, head) with 8 bits into `out` (nothing written in f32).
hipError_t launch_qknorm_rope_q8(const float* q_in, const float* k_in, const float* v_in,
                                 const float* wq, const float* wk, const SeqTable& seqs, int T,
                                 int H, int Hkv, int D, int rope_dim, float base, float eps,
                                 const Q8Rows& out, hipStream_t stream);

// 8-bit quantisation of n_rows rows of len floats: codes, one scale per row and, when
// deq is not null, the dequantised values (code x scale).
hipError_t launch_quant_rows(const float* x, int64_t n_rows, int len, int8_t* codes,
                             float* scales, float* deq, hipStream_t stream);

// prep == nullptr: plain attention on already-normalised Q/K; otherwise the
// fused entry (Q and K normalised and rotated inside the kernel).
hipError_t launch_attn_f32(const float* q, const float* k, const float* v, float* out,
                           const AttnSched& sched, const AttnGeom& geom, int D,
                           const PrepParams* prep, const Partials& part, int n_items,
                           hipStream_t stream);

// Merges the partial results of split items into out (no-op for unsplit ones).
// tile_keys: the key-tile size of the attention kernel that wrote the partials.
hipError_t launch_attn_combine(const Partials& part, float* out, const AttnSched& sched,
                               const AttnGeom& geom, int D, int waves, int tile_keys, int n_items,
                               hipStream_t stream);

// bf16-input / f32-accumulate attention.
// split_qk: scores from bf16 high + low parts of Q and K (PFA_PREC_BF16X3).
// Two kernels: K and V are first converted once into `ws` (bf16 tiles in the byte
// image the attention kernel keeps in LDS), then the attention kernel copies those
// tiles straight into LDS.  ws must hold bf16_workspace_bytes(...) bytes.
// The fused entry adds a rotary table of rope_rows x D/2 (cos, sin) f32 pairs.
constexpr int kBf16TileKeys = 64;
inline size_t bf16_workspace_bytes(int n_tiles, int Hkv, int D, bool split_qk, int rope_rows) {
    return (size_t)n_tiles * Hkv * (split_qk ? 3 : 2) * kBf16TileKeys * D * 2 +
           (size_t)rope_rows * (D / 2) * 8;
}
// Tiles kept across chunk calls (qk_prep_chunk_attn_tiled): sequence s owns the
// cap_tiles tiles of slot s (tile s * cap_tiles + j holds its cache rows 64 j ..), and a
// call re-stages only the tiles its new rows touch, from the f32 cache, together with
// the rotary-table rows of their positions (the table, indexed by position, follows the
// tiles: cap_tiles * 64 rows).  Passed by value to the staging launch.
struct TileAppend {
    int n_seqs;
    int cap_tiles;                 // tiles per sequence slot
    int cum[PFA_MAX_SEQS + 1];     // touched tiles of the sequences before s
    int first[PFA_MAX_SEQS];       // first touched tile of sequence s (slot-local)
    int koff[PFA_MAX_SEQS + 1];    // f32 cache rows of sequence s: koff[s] .. koff[s+1]-1
    int rope_dim;                  // rotated dims of the table rows (0: no table)
    double base;                   // rotary frequency base
};
// prep != nullptr: a fused entry (Q normalised and rotated inside the attention
// kernel; K too, on its way into the tiles, when prep_k -- over a cached prefix
// the cache already holds rotated keys).  app != nullptr: ws is the caller's kept
// tiles (sched.tile_off / n_tiles describe its slots); only the touched tiles are
// staged and no rotary-table launch is needed.  split_qk: the split-score bf16 mode;
// f16: IEEE binary16 operands in the same tile layouts (not with split_qk).
hipError_t launch_attn_bf16(const float* q, const float* k, const float* v, float* out, void* ws,
                            const AttnSched& sched, const AttnGeom& geom, int D, bool split_qk,
                            bool f16, const PrepParams* prep, bool prep_k, const Partials& part,
                            int n_items, hipStream_t stream, const TileAppend* app = nullptr);

// Attention through an 8-bit store, on the bf16 kernel's schedule: the scores are the
// integer dot products of the codes (v_mfma_i32_32x32x32_i8 on int8 K tiles for
// head_dim 128; for 64, codes in bf16 K tiles on the bf16 MFMA -- |code| <= 127 is
// exact in bf16 and the sums of code products stay exact integers in f32) times the
// query and key row scales; V is dequantised (code x scale, rounded to bf16) into bf16
// V tiles.  Workspace: K tiles, V tiles, then 64 key scales per tile and K/V head.
inline size_t q8_tile_bytes(int n_tiles, int Hkv, int D) {
    const size_t kt = (size_t)kBf16TileKeys * D * (D == 128 ? 1 : 2);
    return (size_t)n_tiles * Hkv * (kt + (size_t)kBf16TileKeys * D * 2);
}
inline size_t q8_scale_bytes(int n_tiles, int Hkv) {
    return (size_t)n_tiles * Hkv * kBf16TileKeys * 4;
}
hipError_t launch_attn_q8(const Q8Store& st8, float* out, void* ws, const AttnSched& sched,
                          const AttnGeom& geom, int D, const Partials& part, int n_items,
                          hipStream_t stream);
}  // namespace pfa
