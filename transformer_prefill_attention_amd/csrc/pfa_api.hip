// pfa_api.hip -- the extern "C" entry points of libpfa (declared in
// include/pfa.h): argument validation, the packed-sequence tables and the
// attention work schedule are built on the host, then kernels are enqueued on
// the caller's stream.  Nothing here allocates device memory or synchronises.
//
// Error convention (needle-core v3/model.rs keeps failures recoverable for its
// binding callers: an empty prompt is an empty result and bad shapes come back
// as errors rather than aborts): every problem is reported as a status code
// with a thread-local message, and T == 0 succeeds without a launch.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <vector>

#include "pfa_device.h"
#include "pfa_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

// The f32 tensors are read and written in 16-byte vectors: every (non-null) one must be
// 16-byte aligned, as the header requires.  Checked after the other arguments, just
// before anything is enqueued.
int check_aligned(std::initializer_list<const void*> ptrs) {
    for (const void* p : ptrs)
        if (p && !aligned16(p))
            return fail(PFA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    return 0;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const char* pa = static_cast<const char*>(a);
    const char* pb = static_cast<const char*>(b);
    return pa < pb + nb && pb < pa + na;
}

// Shared shape checks.  Returns PFA_OK or a failure (message set).
int check_geometry(int T, int n_head, int n_head_kv, int head_dim) {
    if (T < 0) return fail(PFA_ERR_INVALID_ARG, "T must be >= 0 (got %d)", T);
    if (n_head <= 0 || n_head_kv <= 0)
        return fail(PFA_ERR_INVALID_ARG, "n_head (%d) and n_head_kv (%d) must be positive", n_head,
                    n_head_kv);
    if (n_head > PFA_MAX_HEADS)
        return fail(PFA_ERR_UNSUPPORTED, "at most %d query heads (got %d)", PFA_MAX_HEADS, n_head);
    if (n_head % n_head_kv)
        return fail(PFA_ERR_INVALID_ARG, "n_head (%d) must be a multiple of n_head_kv (%d)",
                    n_head, n_head_kv);
    if (head_dim <= 0) return fail(PFA_ERR_INVALID_ARG, "head_dim must be positive");
    if (head_dim != 64 && head_dim != 128)
        return fail(PFA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
    const long long elems = (long long)T * std::max(n_head, n_head_kv) * head_dim;
    if (elems >= (1LL << 31))
        return fail(PFA_ERR_UNSUPPORTED, "T * heads * head_dim = %lld exceeds 2^31 - 1", elems);
    return PFA_OK;
}

int check_rope(int head_dim, int rope_dim, float base, float eps) {
    if (rope_dim < 2 || rope_dim > head_dim || (rope_dim & 1))
        return fail(PFA_ERR_INVALID_ARG, "rope_dim must be even with 2 <= rope_dim <= head_dim "
                                         "(got %d, head_dim %d)", rope_dim, head_dim);
    if (!(base > 0.0f) || !std::isfinite(base))
        return fail(PFA_ERR_INVALID_ARG, "rope_freq_base must be finite and > 0");
    if (!(eps >= 0.0f) || !std::isfinite(eps))
        return fail(PFA_ERR_INVALID_ARG, "rms_eps must be finite and >= 0");
    return PFA_OK;
}

// Copies seq_offsets (host) into a kernel-argument table.
int build_seqs(const int32_t* seq_offsets, int n_seqs, int T, pfa::SeqTable& st) {
    if (!seq_offsets) {
        st.n_seqs = 1;
        st.off[0] = st.koff[0] = 0;
        st.off[1] = st.koff[1] = T;
        return PFA_OK;
    }
    if (n_seqs < 1) return fail(PFA_ERR_INVALID_ARG, "n_seqs must be >= 1 (got %d)", n_seqs);
    if (n_seqs > PFA_MAX_SEQS)
        return fail(PFA_ERR_UNSUPPORTED, "at most %d packed sequences (got %d)", PFA_MAX_SEQS,
                    n_seqs);
    if (seq_offsets[0] != 0) return fail(PFA_ERR_INVALID_ARG, "seq_offsets[0] must be 0");
    for (int s = 0; s < n_seqs; ++s)
        if (seq_offsets[s + 1] < seq_offsets[s])
            return fail(PFA_ERR_INVALID_ARG, "seq_offsets must be non-decreasing (index %d)", s);
    if (seq_offsets[n_seqs] != T)
        return fail(PFA_ERR_INVALID_ARG, "seq_offsets[n_seqs] = %d but T = %d",
                    seq_offsets[n_seqs], T);
    st.n_seqs = n_seqs;
    for (int s = 0; s <= n_seqs; ++s) st.off[s] = st.koff[s] = seq_offsets[s];
    return PFA_OK;
}

// Query rows and cache rows of the chunk entry points: each sequence needs at
// least as many cache rows as query rows (its queries are the last ones).
int build_chunk_seqs(const int32_t* q_offsets, const int32_t* kv_offsets, int n_seqs, int T_q,
                     int T_kv, pfa::SeqTable& st) {
    if ((q_offsets == nullptr) != (kv_offsets == nullptr))
        return fail(PFA_ERR_INVALID_ARG, "q_offsets and kv_offsets: both or neither");
    int rc = build_seqs(q_offsets, n_seqs, T_q, st);
    if (rc) return rc;
    pfa::SeqTable kt;
    if ((rc = build_seqs(kv_offsets, n_seqs, T_kv, kt))) return rc;
    for (int s = 0; s < st.n_seqs; ++s)
        if (kt.off[s + 1] - kt.off[s] < st.off[s + 1] - st.off[s])
            return fail(PFA_ERR_INVALID_ARG,
                        "sequence %d has %d cache rows for %d query rows (needs at least as many)",
                        s, kt.off[s + 1] - kt.off[s], st.off[s + 1] - st.off[s]);
    for (int s = 0; s <= st.n_seqs; ++s) st.koff[s] = kt.off[s];
    return PFA_OK;
}

// Work split of a workgroup of `waves` wavefronts for group size g: as many heads
// of the group as divide both g and 4, the other wavefronts take more 32-row
// query blocks.
void choose_geometry(int H, int Hkv, float scale, int causal, int waves, pfa::AttnGeom& geom) {
    const int g = H / Hkv;
    int hpw = 1;
    while (hpw < 4 && g % (hpw * 2) == 0) hpw *= 2;
    geom.H = H;
    geom.Hkv = Hkv;
    geom.g = g;
    geom.hpw = hpw;
    geom.rb = waves / hpw;
    geom.chunks = g / hpw;
    geom.qscale = scale * 1.4426950408889634f;
    geom.causal = causal ? 1 : 0;
    geom.window = 0;
    geom.gate = nullptr;
    geom.gate_per_head = 0;
}

// Longest-first schedule of (sequence, super-block) items.
int build_sched(const pfa::SeqTable& st, int rows_per_item, pfa::AttnSched& sc) {
    sc.n_seqs = st.n_seqs;
    sc.rows_per_item = rows_per_item;
    sc.paired = 0;
    for (int s = 0; s <= st.n_seqs; ++s) {
        sc.off[s] = st.off[s];
        sc.koff[s] = st.koff[s];
    }
    int nsb[PFA_MAX_SEQS];
    int idx[PFA_MAX_SEQS];
    for (int s = 0; s < st.n_seqs; ++s) {
        nsb[s] = (st.off[s + 1] - st.off[s] + rows_per_item - 1) / rows_per_item;
        idx[s] = s;
    }
    std::stable_sort(idx, idx + st.n_seqs, [&](int a, int b) { return nsb[a] > nsb[b]; });
    int n_nonempty = 0;
    for (int s = 0; s < st.n_seqs; ++s) {
        sc.order[s] = idx[s];
        if (nsb[idx[s]] > 0) ++n_nonempty;
    }
    int items = 0;
    sc.n_segs = n_nonempty;
    for (int kk = 0; kk < n_nonempty; ++kk) {
        const int top = nsb[idx[kk]];
        const int next = kk + 1 < n_nonempty ? nsb[idx[kk + 1]] : 0;
        sc.seg_start[kk] = items;
        sc.seg_top[kk] = top;
        items += (kk + 1) * (top - next);
    }
    sc.seg_start[n_nonempty] = items;
    // 64-key tiles of each sequence's key rows in the bf16 workspace
    sc.tile_off[0] = 0;
    for (int s = 0; s < st.n_seqs; ++s)
        sc.tile_off[s + 1] =
            sc.tile_off[s] + (st.koff[s + 1] - st.koff[s] + pfa::kBf16TileKeys - 1) /
                                 pfa::kBf16TileKeys;
    sc.n_tiles = sc.tile_off[st.n_seqs];
    sc.max_len = 0;
    for (int s = 0; s < st.n_seqs; ++s)
        sc.max_len = std::max(sc.max_len, st.koff[s + 1] - st.koff[s]);
    return items;
}

// Everything an attention call launches, decided on the host from its arguments
// (the same for pfa_workspace_bytes and the call itself).
struct Plan {
    pfa::AttnGeom geom;
    pfa::AttnSched sched;
    int items = 0;
    int waves = 0, tile_keys = 0, head_dim = 0;
    size_t tile_bytes = 0;   // bf16: K/V tiles
    size_t table_bytes = 0;  // bf16 fused entry: rotary table (max_len x d/2 pairs)
    size_t krot_bytes = 0;   // f32 fused entry: the normalised, rotated K (T x Hkv x d)
    size_t part_bytes = 0;   // key split: partial results (and merge counters)
    long long counters = 0;  // key split merged in place: arrival counters (else 0)
    // the partial-result parts inside the workspace region at `base`, this call's tag
    pfa::Partials partials(void* base) const;
};

// Tag of one call's merge counters (see pfa::Partials): 1 .. 2^48 - 1, never repeating
// within 2^48 - 1 calls of the process.
unsigned long long next_call_tag() {
    static std::atomic<unsigned long long> tag{0};
    unsigned long long t;
    do {
        t = (tag.fetch_add(1, std::memory_order_relaxed) + 1) & ((1ull << 48) - 1);
    } while (t == 0);
    return t;
}

pfa::Partials Plan::partials(void* base) const {
    if (!part_bytes) return pfa::Partials{nullptr, nullptr, nullptr, 0};
    const long long units = (long long)items * sched.max_chunks * geom.chunks * geom.Hkv;
    return pfa::partials_at(base, (int)units, waves, head_dim, counters,
                            counters ? next_call_tag() : 0);
}

constexpr int kF32TileKeys = 32;
// Compute units of the current device: the workgroups that fill the GPU once are its CUs x
// (2 f32 or 1 bf16 workgroups per CU).  256 (a whole MI355X) when no device is visible, as
// for the size queries on a host without a GPU; a partitioned GPU reports its share.  Read
// once per device.
int device_cus() {
    constexpr int kWholeGpu = 256, kMaxDevices = 64;
    static int cache[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return kWholeGpu;
    }
    int n = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0) {
        (void)hipGetLastError();
        n = kWholeGpu;
    }
    __atomic_store_n(&cache[dev], n, __ATOMIC_RELAXED);
    return n;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Key split: when items x head chunks x K/V heads workgroups cannot fill the GPU's
// workgroup slots (target: 256 CUs x 2 f32 or x 1 bf16 workgroups), cut every
// item's key tiles into chunks of kchunk tiles.  With the longest item at n_max
// tiles, a causal item of n tiles becomes ceil(n / kchunk) units; kchunk = wgs
// n_max / target keeps a causal single sequence near target / 2 + wgs / 2 units, so the
// f32 kernel takes the shortest chunk (from kSplitMinKeys on) whose units still fit the
// target, counted from each item's own tiles.
// Each unit re-reads its Q rows and writes a partial result, so a chunk holds at
// least 128 keys (at T = 512 shorter chunks were 4-12% slower; a chunk of 1024
// new rows over 7168 cached ones, whose items fill only half the slots, gets two:
// 7-24% faster), and an item is cut into at most kMaxKeyChunks chunks (one new row
// over 8191 cached ones ran 8-20% slower in 64 chunks than in 32).
// Items of at most kMergeChunks chunks are merged in place by their last unit, more
// by the combine launch, which spreads the partial results of many chunks over more
// workgroups (256 new rows over 8192 cached keys in 8 chunks: f32 307 us with the
// launch against 325 in place, bf16 71 against 95; in place with up to 4 chunks, f32
// T = 512 / 1024 with 32/8 heads 61 -> 54 / 161 -> 151 us, bf16x3 T = 1024 with 16/8
// heads 63 -> 51 us).
// The bf16 kernel with plain bf16, f16 or 8-bit inputs (short_steps) splits by the
// rule below only when a sequence spans at least kBf16SplitTiles tiles (2048 keys): its
// tile step is short, and below that the fill-the-target chunks lose to the unsplit
// kernel (T = 512 with 32/8 heads: unsplit 32.7 us, split 40.1 in place, 42.3 with the
// combine launch).  Shorter inputs whose items fill at most a quarter of the slots are
// cut in two halves instead (merged in place), when a half is at least 6 tiles or the
// items fill at most an eighth of the slots: measured with 16/8 heads, T = 512 / 768 /
// 1024, plain bf16 32.2 / 38.3 / 44.5 -> 31.2 / 35.4 / 41.2 us, fused entry 46.7 / 53.0
// / 59.7 -> 45.2 / 50.8 / 55.9, 8-bit store 29.6 / 35.8 / 42.2 -> 28.6 / 32.4 / 36.5;
// halves of 4 tiles at T = 512 with 32/8 heads lost (32.8 -> 33.9 us).
constexpr int kMaxKeyChunks = 32;
constexpr int kBf16SplitTiles = 32;
// Shortest key chunk the causally balanced split of the f32 kernel (below) may choose.
// Measured, f32, 32/8 heads of 128: T = 896 / 1024 / 1152 / 1280 split into 10 / 11 / 15 /
// 19-tile chunks instead of 13 / 16 / 21 / 25 ran 0.123 -> 0.101, 0.144 -> 0.111, 0.180 ->
// 0.140 and 0.213 -> 0.171 ms, but T = 768 in 6-tile chunks (192 keys) instead of 9 ran
// 0.092 -> 0.110 ms.  The 16-bit kernel lost at every length tried (bf16x3: T = 1024 in
// 6 tiles of 64 keys instead of 8, +2.6%; T = 1280 in 10 instead of 13, +6%): its units'
// fixed work (eight wavefronts' prologue, partial results, merge) weighs more.
constexpr int kSplitMinKeys = 320;

void choose_split(Plan& p, int head_dim, bool short_steps) {
    p.head_dim = head_dim;
    const long long wgs = (long long)p.items * p.geom.chunks * p.geom.Hkv;
    const int target = (p.waves == 8 ? 1 : 2) * device_cus();
    const int n_max = (p.sched.max_len + p.tile_keys - 1) / p.tile_keys;
    const long long k_min = std::max<long long>((128 + p.tile_keys - 1) / p.tile_keys,
                                                (n_max + kMaxKeyChunks - 1) / kMaxKeyChunks);
    const int n_split = short_steps ? kBf16SplitTiles : 2;  // fewest tiles worth splitting
    int kchunk = 0;
    if (wgs < target && n_max >= n_split) {
        // As if every item spanned n_max tiles: the chunk length that fills the target
        const long long k_full = std::max(k_min, (wgs * n_max + target - 1) / target);
        // The items' own tile counts (under the causal mask a sequence's early query blocks
        // see few keys, so k_full leaves most units short and half the slots idle): the
        // shortest chunk length from k_min on whose non-empty units still fit the target,
        // and, where k_full's chunks can be merged in place, no more chunks than that takes.
        // Chunks stay at least kSplitMinKeys long; the 16-bit kernels keep k_full (see
        // kSplitMinKeys).  Computed without the window, as the workspace query is.
        const long long min_tiles = (kSplitMinKeys + p.tile_keys - 1) / p.tile_keys;
        long long c_lo = std::max(k_min, min_tiles);
        if ((n_max + k_full - 1) / k_full <= pfa::kMergeChunks)
            c_lo = std::max(c_lo, (long long)(n_max + pfa::kMergeChunks - 1) / pfa::kMergeChunks);
        if (p.waves == 8) c_lo = k_full;
        p.sched.kchunk = 0;
        p.sched.max_chunks = 1;
        std::vector<int> tiles((size_t)p.items);
        for (int i = 0; i < p.items; ++i) {
            const pfa::WorkItem w =
                pfa::decode_item(p.sched, p.geom, i * p.geom.chunks * p.geom.Hkv);
            const pfa::KeyRange r = pfa::item_key_range(p.sched, p.geom, w, p.tile_keys);
            tiles[(size_t)i] = r.n_tiles - r.t_first;
        }
        long long k = k_full;
        for (long long c = c_lo; c < k_full; ++c) {
            long long units = 0;
            for (const int t : tiles) units += (t + c - 1) / c;
            if (units * p.geom.chunks * p.geom.Hkv <= target) {
                k = c;
                break;
            }
        }
        kchunk = (int)k;
        if (kchunk >= n_max) kchunk = 0;
    } else if (short_steps && n_max >= 8 && wgs * 4 <= target) {
        const int half = (n_max + 1) / 2;  // two chunks an item (see kBf16SplitTiles)
        if (half >= 6 || wgs * 8 <= target) kchunk = half;
    }
    p.sched.kchunk = kchunk;
    p.sched.max_chunks = kchunk ? (n_max + kchunk - 1) / kchunk : 1;
    const long long units =
        (long long)p.items * p.sched.max_chunks * p.geom.chunks * p.geom.Hkv;
    p.counters = kchunk && p.sched.max_chunks <= pfa::kMergeChunks
                     ? (long long)p.items * p.geom.chunks * p.geom.Hkv
                     : 0;
    p.part_bytes = kchunk ? pfa::partials_bytes((int)units, p.waves, head_dim, p.counters) : 0;
}

// Paired items for the f32 kernel (AttnSched::paired): each workgroup takes item j and
// item n - 1 - j of one causal sequence, so all workgroups visit the same number of key
// tiles.  That balances the CUs when the paired workgroups divide evenly over the CUs (256
// on MI355X) with at most two per CU, or fill whole rounds of two per CU (every later
// round then starts as the previous one's equal-length pairs end): measured at 8B-like
// heads, T = 2048 0.404 -> 0.313 ms, T = 4096 1.197 -> 1.080 ms, T = 8192 (two rounds)
// 4.13 -> 4.08 ms (fused entry 4.21 -> 4.14), T = 12288 and 16384 -1%; T = 3072 (384
// workgroups, one or two per CU) ran 22% slower and packed sequences of unequal length 7%
// slower.  Plain prefill of one sequence only, no key split, no window.  one_round: also
// when the paired grid is at most one workgroup per CU (in place of a key split, below).
bool pair_items(const Plan& p, const pfa::SeqTable& st, int causal, int window, bool chunk,
                bool one_round) {
    if (!causal || window > 0 || chunk || st.n_seqs != 1 || p.sched.max_chunks != 1 ||
        p.items < 2)
        return false;
    const long long wgs = (long long)(p.items + 1) / 2 * p.geom.chunks * p.geom.Hkv;
    const int cus = device_cus();
    return (wgs % cus == 0 && wgs <= 2 * cus) || wgs % (2 * cus) == 0 ||
           (one_round && wgs <= cus);
}

// Key tiles of the longest pair (items j and n - 1 - j; the middle item of an odd count
// alone), from the items' own tile counts.
static long long longest_pair_tiles(const Plan& p) {
    pfa::AttnSched sc = p.sched;
    sc.kchunk = 0;
    sc.max_chunks = 1;
    auto tiles = [&](int i) {
        const pfa::WorkItem w = pfa::decode_item(sc, p.geom, i * p.geom.chunks * p.geom.Hkv);
        const pfa::KeyRange r = pfa::item_key_range(sc, p.geom, w, p.tile_keys);
        return (long long)(r.n_tiles - r.t_first);
    };
    long long best = 0;
    for (int j = 0; j < (p.items + 1) / 2; ++j) {
        const int k = p.items - 1 - j;
        best = std::max(best, tiles(j) + (k != j ? tiles(k) : 0));
    }
    return best;
}

// Geometry, schedule, key split and workspace parts of one attention call.
int make_plan(const pfa::SeqTable& st, int n_head, int n_head_kv, int head_dim, float scale,
              int causal, int precision, Plan& p) {
    const bool bf16 = precision != PFA_PREC_F32;
    // the bf16 kernel runs 8 wavefronts per workgroup, the f32 one 4
    p.waves = bf16 ? 8 : 4;
    p.tile_keys = bf16 ? pfa::kBf16TileKeys : kF32TileKeys;
    choose_geometry(n_head, n_head_kv, scale, causal, p.waves, p.geom);
    p.items = build_sched(st, 32 * p.geom.rb, p.sched);
    // plain bf16 and f16 (and the 8-bit kernels, which plan as bf16): short tile steps
    choose_split(p, head_dim, precision == PFA_PREC_BF16 || precision == PFA_PREC_F16);
    if ((long long)p.items * p.sched.max_chunks * p.geom.chunks * p.geom.Hkv >= (1LL << 31))
        return fail(PFA_ERR_UNSUPPORTED, "grid too large");
    if (bf16) {
        p.tile_bytes = pfa::bf16_workspace_bytes(p.sched.n_tiles, n_head_kv, head_dim,
                                                 precision == PFA_PREC_BF16X3, 0);
        p.table_bytes = pfa::bf16_workspace_bytes(0, n_head_kv, head_dim, false, p.sched.max_len);
    } else {
        p.krot_bytes = (size_t)st.off[st.n_seqs] * n_head_kv * head_dim * 4;
    }
    return PFA_OK;
}

// Workspace bytes ahead of the partial results: the bf16 K/V tiles (+ the rotary
// table when Q is prepared in the kernel), or for the f32 fused entry the rotated
// K unless it goes to the caller's k_rot_out (over a cached prefix it goes to the
// cache instead).
size_t prep_part_bytes(const Plan& p, bool bf16, bool prep_q, bool krot_in_ws) {
    if (bf16) return p.tile_bytes + (prep_q ? p.table_bytes : 0);
    return krot_in_ws ? p.krot_bytes : 0;
}

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess)
        return fail(PFA_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
    return PFA_OK;
}

}  // namespace

extern "C" {

const char* pfa_last_error(void) { return g_err; }

const char* pfa_version(void) {
    return "pfa 0.5 (gfx950; f32 and bf16 MFMA attention, prefill and chunks over a cached prefix, "
           "8-bit quantised sessions)";
}

static bool known_precision(int precision) {
    return precision == PFA_PREC_F32 || precision == PFA_PREC_BF16 ||
           precision == PFA_PREC_BF16X3 || precision == PFA_PREC_F16;
}
static int bad_precision(int precision) {
    return fail(PFA_ERR_INVALID_ARG, "precision must be PFA_PREC_F32, PFA_PREC_BF16, "
                                     "PFA_PREC_BF16X3 or PFA_PREC_F16 (got %d)", precision);
}

static size_t workspace_for(const pfa::SeqTable& st, int n_head, int n_head_kv, int head_dim,
                            int precision, bool prep_q, bool krot_in_ws, bool tiled = false) {
    if (!known_precision(precision)) {
        bad_precision(precision);
        return 0;
    }
    Plan p;
    if (make_plan(st, n_head, n_head_kv, head_dim, 1.0f, 1, precision, p)) return 0;
    if (p.items == 0) return 0;
    const size_t base = tiled ? 0 : prep_part_bytes(p, precision != PFA_PREC_F32, prep_q, krot_in_ws);
    return p.part_bytes ? align256(base) + p.part_bytes : base;
}

size_t pfa_workspace_bytes(const int32_t* seq_offsets, int n_seqs, int T, int n_head,
                           int n_head_kv, int head_dim, int precision, int fused) {
    g_err[0] = 0;
    if (check_geometry(T, n_head, n_head_kv, head_dim)) return 0;
    if (T == 0) return 0;
    pfa::SeqTable st;
    if (build_seqs(seq_offsets, n_seqs, T, st)) return 0;
    return workspace_for(st, n_head, n_head_kv, head_dim, precision, fused != 0,
                         fused != 0 && precision == PFA_PREC_F32);
}

size_t pfa_chunk_workspace_bytes(const int32_t* q_offsets, const int32_t* kv_offsets, int n_seqs,
                                 int T_q, int T_kv, int n_head, int n_head_kv, int head_dim,
                                 int precision, int fused) {
    g_err[0] = 0;
    if (check_geometry(T_q, n_head, n_head_kv, head_dim) ||
        check_geometry(T_kv, n_head, n_head_kv, head_dim))
        return 0;
    if (T_q == 0) return 0;
    pfa::SeqTable st;
    if (build_chunk_seqs(q_offsets, kv_offsets, n_seqs, T_q, T_kv, st)) return 0;
    if (fused == 2 && precision == PFA_PREC_F32) {
        fail(PFA_ERR_INVALID_ARG, "qk_prep_chunk_attn_tiled takes PFA_PREC_BF16, "
                                  "PFA_PREC_BF16X3 or PFA_PREC_F16");
        return 0;
    }
    return workspace_for(st, n_head, n_head_kv, head_dim, precision, fused != 0, false,
                         fused == 2);
}

size_t pfa_kv_tiles_bytes(int n_slots, int max_rows, int n_head_kv, int head_dim, int precision) {
    g_err[0] = 0;
    if (n_slots < 1 || n_slots > PFA_MAX_SEQS) {
        fail(PFA_ERR_INVALID_ARG, "n_slots must be 1..%d (got %d)", PFA_MAX_SEQS, n_slots);
        return 0;
    }
    if (max_rows < 1) {
        fail(PFA_ERR_INVALID_ARG, "max_rows must be >= 1 (got %d)", max_rows);
        return 0;
    }
    if (check_geometry(max_rows, n_head_kv, n_head_kv, head_dim)) return 0;
    if (precision != PFA_PREC_BF16 && precision != PFA_PREC_BF16X3 && precision != PFA_PREC_F16) {
        fail(PFA_ERR_INVALID_ARG,
             "kv_tiles are for PFA_PREC_BF16, PFA_PREC_BF16X3 or PFA_PREC_F16 (got %d)",
             precision);
        return 0;
    }
    const int cap = (max_rows + pfa::kBf16TileKeys - 1) / pfa::kBf16TileKeys;
    return pfa::bf16_workspace_bytes(n_slots * cap, n_head_kv, head_dim,
                                     precision == PFA_PREC_BF16X3, cap * pfa::kBf16TileKeys);
}

int qknorm_rope(const float* q_in, const float* k_in, float* q_out, float* k_out,
                const float* q_norm_w, const float* k_norm_w, const int32_t* seq_offsets,
                int n_seqs, int T, int n_head, int n_head_kv, int head_dim, int rope_dim,
                float rope_freq_base, float rms_eps, void* stream) {
    g_err[0] = 0;
    int rc = check_geometry(T, n_head, n_head_kv, head_dim);
    if (rc) return rc;
    if ((rc = check_rope(head_dim, rope_dim, rope_freq_base, rms_eps))) return rc;
    if (T == 0) return PFA_OK;
    if (!q_in || !k_in || !q_out || !k_out || !q_norm_w || !k_norm_w)
        return fail(PFA_ERR_INVALID_ARG, "null tensor pointer");
    const size_t qb = (size_t)T * n_head * head_dim * 4, kb = (size_t)T * n_head_kv * head_dim * 4;
    if (q_out != q_in && overlaps(q_out, qb, q_in, qb))
        return fail(PFA_ERR_INVALID_ARG, "q_out partially overlaps q_in");
    if (k_out != k_in && overlaps(k_out, kb, k_in, kb))
        return fail(PFA_ERR_INVALID_ARG, "k_out partially overlaps k_in");
    if (overlaps(q_out, qb, k_in, kb) || overlaps(q_out, qb, k_out, kb) ||
        overlaps(k_out, kb, q_in, qb))
        return fail(PFA_ERR_INVALID_ARG, "Q and K buffers overlap");
    pfa::SeqTable st;
    if ((rc = build_seqs(seq_offsets, n_seqs, T, st))) return rc;
    if ((rc = check_aligned({q_in, k_in, q_out, k_out, q_norm_w, k_norm_w}))) return rc;
    return hip_status(pfa::launch_qknorm_rope(q_in, k_in, q_out, k_out, nullptr, nullptr,
                                              q_norm_w, k_norm_w, st, T,
                                              n_head, n_head_kv, head_dim, rope_dim,
                                              rope_freq_base, rms_eps, (hipStream_t)stream),
                      "qknorm_rope launch");
}

// How an attention call gets its K: as given (plain prefill, or a cache for the
// chunk entry), prepared from raw rows into k_rot_out / the workspace (fused
// prefill), or prepared from the new rows into the caller's cache (fused chunk; the
// tiled one also keeps the cache's bf16 tiles in the caller's kv_tiles across calls).
enum class Mode { kPlain, kFused, kChunk, kChunkFused, kChunkTiled };

static int check_attn(float scale, int precision) {
    if (!std::isfinite(scale)) return fail(PFA_ERR_INVALID_ARG, "scale must be finite");
    if (!known_precision(precision)) return bad_precision(precision);
    return PFA_OK;
}

// Everything an attention call of the prefill / chunk entries decides on the host: the
// geometry, schedule and key split (make_plan), whether the f32 key split is dropped for
// want of workspace, paired items, and the workspace parts.  The entry points and the
// plan report (pfa_attn_plan, pfa_attn_units) both come here, so they cannot disagree.
struct CallPlan {
    Plan p;
    bool krot_in_ws = false;  // f32 fused prefill without k_rot_out: rotated K in the workspace
    size_t base = 0;          // workspace bytes before the partial results
    size_t part_off = 0;      // offset of the partial results
    size_t need = 0;          // workspace bytes the call uses
};

// ws_bytes: the workspace the call is given (0 when none).
static int plan_call(Mode mode, const pfa::SeqTable& st, int n_head, int n_head_kv, int head_dim,
                     float scale, int causal, int window, int precision, bool has_k_rot_out,
                     size_t ws_bytes, CallPlan& cp) {
    Plan& p = cp.p;
    int rc = make_plan(st, n_head, n_head_kv, head_dim, scale, causal, precision, p);
    if (rc) return rc;
    p.geom.window = window;
    const bool bf16 = precision != PFA_PREC_F32;
    const bool tiled = mode == Mode::kChunkTiled;
    const bool prep = mode == Mode::kFused || mode == Mode::kChunkFused || tiled;
    const bool chunk = mode == Mode::kChunk || mode == Mode::kChunkFused || tiled;
    // workspace parts: [bf16 K/V tiles + rotary table (Q prepared in the kernel), or f32
    // rotated K (fused prefill without k_rot_out)][partials, key split]; the tiled chunk
    // entry keeps its tiles and table in kv_tiles, so only the partials remain
    // f32, one causal sequence, no window: paired items (one workgroup per CU) in place of
    // a key split whose chunks are long, i.e. when a pair spans fewer tiles than two chunks
    // (measured, 32/8 heads of 128: T = 1536 / 1792, chunks of 32 / 48 tiles against pairs of
    // 49 / 57, 0.337 -> 0.241 and 0.485 -> 0.279 ms; T = 896 / 1024 / 1280, chunks of 10 /
    // 11 / 19 against pairs of 29 / 33 / 41, the split stays faster: 0.101 / 0.111 / 0.171
    // against 0.148 / 0.167 / 0.203 ms).  The size queries still count the split's partial
    // results.  Only chunks of at least kSplitMinKeys (the lengths measured).  A chunk call
    // over no cached rows is prefill and is planned as such, so that its results stay
    // gqa_prefill_attn's bit for bit.
    const bool as_prefill = !chunk || (st.n_seqs == 1 && st.koff[1] == st.off[1]);
    bool pairs_for_split = false;
    if (!bf16 && p.sched.max_chunks > 1 && causal && window == 0 && as_prefill &&
        st.n_seqs == 1 && p.items >= 2 && (long long)p.sched.kchunk * p.tile_keys >= kSplitMinKeys &&
        (long long)(p.items + 1) / 2 * p.geom.chunks * p.geom.Hkv <= device_cus() &&
        longest_pair_tiles(p) < 2LL * p.sched.kchunk) {
        p.sched.kchunk = 0;
        p.sched.max_chunks = 1;
        p.part_bytes = 0;
        p.counters = 0;
        pairs_for_split = true;
    }
    cp.krot_in_ws = mode == Mode::kFused && !bf16 && !has_k_rot_out;
    cp.base = tiled ? 0 : prep_part_bytes(p, bf16, prep, cp.krot_in_ws);
    cp.part_off = p.part_bytes ? align256(cp.base) : cp.base;
    if (!bf16 && p.part_bytes && ws_bytes < cp.part_off + p.part_bytes) {
        // f32 runs without the key split when the caller gives no (or too small a) workspace
        p.sched.kchunk = 0;
        p.sched.max_chunks = 1;
        p.part_bytes = 0;
        p.counters = 0;
    }
    cp.need = p.part_bytes ? cp.part_off + p.part_bytes : cp.base;
    p.sched.paired =
        !bf16 && pair_items(p, st, causal, window, !as_prefill, pairs_for_split) ? 1 : 0;
    return PFA_OK;
}

static int attn_common(Mode mode, const float* q, const float* k, const float* v, float* out,
                       float* k_cache, float* v_cache, const float* gate, int gate_per_head,
                       const pfa::SeqTable& st, int n_head, int n_head_kv, int head_dim,
                       float scale, int causal, int window, int precision,
                       const pfa::PrepParams* prep, void* workspace, size_t workspace_bytes,
                       void* stream, void* kv_tiles = nullptr, int cap_tiles = 0) {
    const int T_q = st.off[st.n_seqs], T_kv = st.koff[st.n_seqs];
    if (T_q == 0) return PFA_OK;
    const bool tiled = mode == Mode::kChunkTiled;
    const bool chunk_fused = mode == Mode::kChunkFused || tiled;
    if (!q || !k || !v || !out || (chunk_fused && (!k_cache || !v_cache)))
        return fail(PFA_ERR_INVALID_ARG, "null tensor pointer");
    // bytes of Q / out, of the K and V the call reads, and of the caches
    const size_t qb = (size_t)T_q * n_head * head_dim * 4;
    const size_t kb = (size_t)(mode == Mode::kChunk ? T_kv : T_q) * n_head_kv * head_dim * 4;
    const size_t cb = (size_t)T_kv * n_head_kv * head_dim * 4;
    if (overlaps(out, qb, q, qb) || overlaps(out, qb, k, kb) || overlaps(out, qb, v, kb))
        return fail(PFA_ERR_INVALID_ARG, "out must not overlap q, k or v");
    const size_t gb = gate ? (size_t)T_q * n_head * (gate_per_head ? 1 : head_dim) * 4 : 0;
    if (gate && overlaps(gate, gb, out, qb))
        return fail(PFA_ERR_INVALID_ARG, "gate must not overlap out");
    if (prep && prep->k_rot_out &&
        (overlaps(prep->k_rot_out, kb, q, qb) || overlaps(prep->k_rot_out, kb, k, kb) ||
         overlaps(prep->k_rot_out, kb, v, kb) || overlaps(prep->k_rot_out, kb, out, qb)))
        return fail(PFA_ERR_INVALID_ARG, "k_rot_out must not overlap the inputs or out");
    if (chunk_fused) {
        const void* others[4] = {q, k, v, out};
        const size_t sizes[4] = {qb, kb, kb, qb};
        for (int i = 0; i < 4; ++i)
            if (overlaps(k_cache, cb, others[i], sizes[i]) ||
                overlaps(v_cache, cb, others[i], sizes[i]))
                return fail(PFA_ERR_INVALID_ARG,
                            "k_cache / v_cache must not overlap q, k, v or out");
        if (overlaps(k_cache, cb, v_cache, cb))
            return fail(PFA_ERR_INVALID_ARG, "k_cache and v_cache overlap");
    }
    // the kept tiles (tiled chunk entry): slots of cap_tiles tiles, then the rotary table
    const size_t tb = tiled ? pfa::bf16_workspace_bytes(st.n_seqs * cap_tiles, n_head_kv, head_dim,
                                                        precision == PFA_PREC_BF16X3,
                                                        cap_tiles * pfa::kBf16TileKeys)
                            : 0;
    if (tiled) {
        if (!kv_tiles) return fail(PFA_ERR_INVALID_ARG, "null kv_tiles");
        if (reinterpret_cast<uintptr_t>(kv_tiles) % 256)
            return fail(PFA_ERR_INVALID_ARG, "kv_tiles must be 256-byte aligned");
        for (int s = 0; s < st.n_seqs; ++s)
            if (st.koff[s + 1] - st.koff[s] > cap_tiles * pfa::kBf16TileKeys)
                return fail(PFA_ERR_INVALID_ARG,
                            "sequence %d has %d cache rows, more than max_rows (%d, in tiles of "
                            "%d)", s, st.koff[s + 1] - st.koff[s],
                            cap_tiles * pfa::kBf16TileKeys, pfa::kBf16TileKeys);
        const void* others[7] = {q, k, v, out, k_cache, v_cache, gate};
        const size_t sizes[7] = {qb, kb, kb, qb, cb, cb, gate ? gb : 0};
        for (int i = 0; i < 7; ++i)
            if (others[i] && overlaps(kv_tiles, tb, others[i], sizes[i]))
                return fail(PFA_ERR_INVALID_ARG, "kv_tiles must not overlap the other tensors");
    }
    CallPlan cp;
    int rc;
    if ((rc = plan_call(mode, st, n_head, n_head_kv, head_dim, scale, causal, window, precision,
                        prep && prep->k_rot_out, workspace ? workspace_bytes : 0, cp)))
        return rc;
    Plan& p = cp.p;
    if (p.items == 0) return PFA_OK;
    p.geom.gate = gate;
    p.geom.gate_per_head = gate_per_head ? 1 : 0;
    const bool bf16 = precision != PFA_PREC_F32;
    const size_t part_off = cp.part_off, need = cp.need;
    if (need > 0) {
        if (!workspace)
            return fail(PFA_ERR_INVALID_ARG, "precision %d needs a workspace (%zu bytes)",
                        precision, need);
        if (workspace_bytes < need)
            return fail(PFA_ERR_INVALID_ARG, "workspace of %zu bytes, %zu needed",
                        workspace_bytes, need);
        if (reinterpret_cast<uintptr_t>(workspace) % 256)
            return fail(PFA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
        if (overlaps(workspace, need, q, qb) || overlaps(workspace, need, k, kb) ||
            overlaps(workspace, need, v, kb) || overlaps(workspace, need, out, qb) ||
            (prep && prep->k_rot_out && overlaps(workspace, need, prep->k_rot_out, kb)) ||
            (chunk_fused &&
             (overlaps(workspace, need, k_cache, cb) || overlaps(workspace, need, v_cache, cb))) ||
            (tiled && overlaps(workspace, need, kv_tiles, tb)))
            return fail(PFA_ERR_INVALID_ARG, "workspace must not overlap the tensors");
    }
    const pfa::Partials part = p.partials(static_cast<char*>(workspace) + part_off);
    if ((rc = check_aligned({q, k, v, out, k_cache, v_cache, gate, prep ? prep->wq : nullptr,
                             prep ? prep->wk : nullptr, prep ? prep->k_rot_out : nullptr})))
        return rc;
    const char* what = prep ? (tiled         ? "qk_prep_chunk_attn_tiled launch"
                               : chunk_fused ? "qk_prep_chunk_attn launch"
                                             : "qk_prep_attn launch")
                            : (mode == Mode::kChunk ? "gqa_chunk_attn launch"
                                                    : "gqa_prefill_attn launch");
    const float* k_attn = k;
    const float* v_attn = v;
    if (chunk_fused) {
        // the new rows: K normalised and rotated at their positions, K and V written
        // to the last rows of each sequence's cache range; attention reads the caches
        if ((rc = hip_status(pfa::launch_qknorm_rope(nullptr, k, nullptr, k_cache, v, v_cache,
                                                     prep->wq, prep->wk, st, T_q, 0, n_head_kv,
                                                     head_dim, prep->rope_dim, (float)prep->base,
                                                     prep->eps, (hipStream_t)stream),
                             what)))
            return rc;
        k_attn = k_cache;
        v_attn = v_cache;
    }
    if (tiled) {
        // the attention kernel reads sequence s's tiles from slot s of kv_tiles; the
        // staging launch re-stages the tiles holding this call's new rows (the first
        // of them may hold earlier rows too: they come from the cache like the rest)
        pfa::TileAppend app{};
        app.n_seqs = st.n_seqs;
        app.cap_tiles = cap_tiles;
        app.rope_dim = prep->rope_dim;
        app.base = prep->base;
        constexpr int TK = pfa::kBf16TileKeys;
        for (int s = 0; s <= st.n_seqs; ++s) {
            p.sched.tile_off[s] = s * cap_tiles;
            app.koff[s] = st.koff[s];
        }
        p.sched.n_tiles = st.n_seqs * cap_tiles;
        app.cum[0] = 0;
        for (int s = 0; s < st.n_seqs; ++s) {
            const int kv_len = st.koff[s + 1] - st.koff[s], n_new = st.off[s + 1] - st.off[s];
            app.first[s] = (kv_len - n_new) / TK;
            app.cum[s + 1] = app.cum[s] + (n_new > 0 ? (kv_len + TK - 1) / TK - app.first[s] : 0);
        }
        return hip_status(pfa::launch_attn_bf16(q, k_attn, v_attn, out, kv_tiles, p.sched, p.geom,
                                                head_dim, precision == PFA_PREC_BF16X3,
                                                precision == PFA_PREC_F16, prep, false, part,
                                                p.items, (hipStream_t)stream, &app),
                          what);
    }
    if (bf16)
        return hip_status(pfa::launch_attn_bf16(q, k_attn, v_attn, out, workspace, p.sched, p.geom,
                                                head_dim, precision == PFA_PREC_BF16X3,
                                                precision == PFA_PREC_F16, prep,
                                                mode == Mode::kFused, part, p.items,
                                                (hipStream_t)stream),
                          what);
    if (mode == Mode::kFused) {
        // f32 fused prefill: K is normalised and rotated once, by the QK-norm + RoPE
        // kernel over the K rows alone, into k_rot_out or the workspace; the
        // attention kernel then prepares only its own Q rows
        float* krot = prep->k_rot_out ? prep->k_rot_out : static_cast<float*>(workspace);
        if ((rc = hip_status(pfa::launch_qknorm_rope(nullptr, k, nullptr, krot, nullptr, nullptr,
                                                     prep->wq, prep->wk, st, T_q, 0, n_head_kv,
                                                     head_dim, prep->rope_dim,
                                                     (float)prep->base, prep->eps,
                                                     (hipStream_t)stream),
                             what)))
            return rc;
        k_attn = krot;
    }
    return hip_status(pfa::launch_attn_f32(q, k_attn, v_attn, out, p.sched, p.geom, head_dim, prep,
                                           part, p.items, (hipStream_t)stream),
                      what);
}

int gqa_prefill_attn(const float* q, const float* k, const float* v, float* out,
                     const int32_t* seq_offsets, int n_seqs, int T, int n_head, int n_head_kv,
                     int head_dim, float scale, int causal, int precision, void* workspace,
                     size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    int rc = check_geometry(T, n_head, n_head_kv, head_dim);
    if (rc || (rc = check_attn(scale, precision))) return rc;
    if (T == 0) return PFA_OK;
    pfa::SeqTable st;
    if ((rc = build_seqs(seq_offsets, n_seqs, T, st))) return rc;
    return attn_common(Mode::kPlain, q, k, v, out, nullptr, nullptr, nullptr, 0, st, n_head,
                       n_head_kv, head_dim, scale, causal, 0, precision, nullptr, workspace,
                       workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// gqa_prefill_attn_noalloc: gqa_prefill_attn for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  Its workspace is this library-owned device array (each GPU the library
// runs on holds one copy until the process ends); it is resolved to a device address
// once per device with hipGetSymbolAddress, and only that address reaches the kernels.
// Nothing in it needs clearing: the staging kernels write every tile they later read, the
// key split writes every partial result before it is merged, and the in-place merge's
// arrival counters are tagged per call (a value left by another call counts as none) and
// left 0.  Calls that overlap on one GPU share the array and race.
namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on the current device (nullptr and a message on failure).
void* scratch_address() {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        fail(PFA_ERR_HIP, "gqa_prefill_attn_noalloc: no usable current device (%s)",
             hipGetErrorString(e));
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            fail(PFA_ERR_HIP, "gqa_prefill_attn_noalloc: hipGetSymbolAddress: HIP error %d (%s)",
                 (int)e, hipGetErrorString(e));
            return nullptr;
        }
        addr[dev] = p;
    }
    return addr[dev];
}

}  // namespace

extern "C" {

size_t pfa_noalloc_scratch_bytes(void) { return kScratchBytes; }

int gqa_prefill_attn_noalloc(const float* q, const float* k, const float* v, float* out,
                             const int32_t* seq_offsets, int n_seqs, int T, int n_head,
                             int n_head_kv, int head_dim, float scale, int causal, int precision,
                             void* stream) {
    g_err[0] = 0;
    int rc = check_geometry(T, n_head, n_head_kv, head_dim);
    if (rc || (rc = check_attn(scale, precision))) return rc;
    if (T == 0) return PFA_OK;
    pfa::SeqTable st;
    if ((rc = build_seqs(seq_offsets, n_seqs, T, st))) return rc;
    // the workspace gqa_prefill_attn would use with room for everything (the same plan)
    CallPlan cp;
    if ((rc = plan_call(Mode::kPlain, st, n_head, n_head_kv, head_dim, scale, causal, 0,
                        precision, false, SIZE_MAX, cp)))
        return rc;
    if (cp.p.items == 0) return PFA_OK;
    if (cp.need > kScratchBytes)
        return fail(PFA_ERR_UNSUPPORTED,
                    "gqa_prefill_attn_noalloc: this call needs %zu bytes of workspace, more than "
                    "the library's %zu-byte device array (use gqa_prefill_attn with a workspace)",
                    cp.need, kScratchBytes);
    void* ws = cp.need ? scratch_address() : nullptr;
    if (cp.need && !ws) return PFA_ERR_HIP;
    return attn_common(Mode::kPlain, q, k, v, out, nullptr, nullptr, nullptr, 0, st, n_head,
                       n_head_kv, head_dim, scale, causal, 0, precision, nullptr, ws,
                       cp.need ? kScratchBytes : 0, stream);
}

int qk_prep_attn(const float* q, const float* k, const float* v, float* out,
                 const float* q_norm_w, const float* k_norm_w, const int32_t* seq_offsets,
                 int n_seqs, int T, int n_head, int n_head_kv, int head_dim, int rope_dim,
                 float rope_freq_base, float rms_eps, float scale, int causal, int precision,
                 float* k_rot_out, void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    int rc = check_geometry(T, n_head, n_head_kv, head_dim);
    if (rc || (rc = check_attn(scale, precision))) return rc;
    if ((rc = check_rope(head_dim, rope_dim, rope_freq_base, rms_eps))) return rc;
    if (T == 0) return PFA_OK;
    if (!q_norm_w || !k_norm_w) return fail(PFA_ERR_INVALID_ARG, "null norm weights");
    pfa::SeqTable st;
    if ((rc = build_seqs(seq_offsets, n_seqs, T, st))) return rc;
    pfa::PrepParams prep{q_norm_w, k_norm_w, k_rot_out, rope_dim, rms_eps,
                         (double)rope_freq_base};
    return attn_common(Mode::kFused, q, k, v, out, nullptr, nullptr, nullptr, 0, st, n_head,
                       n_head_kv, head_dim, scale, causal, 0, precision, &prep, workspace,
                       workspace_bytes, stream);
}

static int check_window(int window, int causal) {
    if (window < 0) return fail(PFA_ERR_INVALID_ARG, "window must be >= 0 (got %d)", window);
    if (window > 0 && !causal)
        return fail(PFA_ERR_INVALID_ARG, "a sliding window needs causal attention");
    return PFA_OK;
}

int gqa_chunk_attn(const float* q, const float* k_cache, const float* v_cache, float* out,
                   const float* gate, int gate_per_head, const int32_t* q_offsets,
                   const int32_t* kv_offsets, int n_seqs, int T_q, int T_kv, int n_head,
                   int n_head_kv, int head_dim, float scale, int causal, int window,
                   int precision, void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    int rc = check_geometry(T_q, n_head, n_head_kv, head_dim);
    if (rc || (rc = check_geometry(T_kv, n_head, n_head_kv, head_dim))) return rc;
    if ((rc = check_attn(scale, precision)) || (rc = check_window(window, causal))) return rc;
    pfa::SeqTable st;
    if ((rc = build_chunk_seqs(q_offsets, kv_offsets, n_seqs, T_q, T_kv, st))) return rc;
    if (T_q == 0) return PFA_OK;
    return attn_common(Mode::kChunk, q, k_cache, v_cache, out, nullptr, nullptr, gate,
                       gate_per_head, st, n_head, n_head_kv, head_dim, scale, causal, window,
                       precision, nullptr, workspace, workspace_bytes, stream);
}

int qk_prep_chunk_attn(const float* q, const float* k, const float* v, float* out,
                       const float* gate, int gate_per_head, const float* q_norm_w,
                       const float* k_norm_w, float* k_cache, float* v_cache,
                       const int32_t* q_offsets, const int32_t* kv_offsets,
                       int n_seqs, int T_q, int T_kv, int n_head, int n_head_kv, int head_dim,
                       int rope_dim, float rope_freq_base, float rms_eps, float scale,
                       int causal, int window, int precision, void* workspace,
                       size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    int rc = check_geometry(T_q, n_head, n_head_kv, head_dim);
    if (rc || (rc = check_geometry(T_kv, n_head, n_head_kv, head_dim))) return rc;
    if ((rc = check_attn(scale, precision)) || (rc = check_window(window, causal))) return rc;
    if ((rc = check_rope(head_dim, rope_dim, rope_freq_base, rms_eps))) return rc;
    pfa::SeqTable st;
    if ((rc = build_chunk_seqs(q_offsets, kv_offsets, n_seqs, T_q, T_kv, st))) return rc;
    if (T_q == 0) return PFA_OK;
    if (!q_norm_w || !k_norm_w) return fail(PFA_ERR_INVALID_ARG, "null norm weights");
    pfa::PrepParams prep{q_norm_w, k_norm_w, nullptr, rope_dim, rms_eps, (double)rope_freq_base};
    return attn_common(Mode::kChunkFused, q, k, v, out, k_cache, v_cache, gate, gate_per_head,
                       st, n_head, n_head_kv, head_dim, scale, causal, window, precision, &prep,
                       workspace, workspace_bytes, stream);
}

int qk_prep_chunk_attn_tiled(const float* q, const float* k, const float* v, float* out,
                             const float* gate, int gate_per_head, const float* q_norm_w,
                             const float* k_norm_w, float* k_cache, float* v_cache,
                             void* kv_tiles, int max_rows, const int32_t* q_offsets,
                             const int32_t* kv_offsets, int n_seqs, int T_q, int T_kv,
                             int n_head, int n_head_kv, int head_dim, int rope_dim,
                             float rope_freq_base, float rms_eps, float scale, int causal,
                             int window, int precision, void* workspace, size_t workspace_bytes,
                             void* stream) {
    g_err[0] = 0;
    int rc = check_geometry(T_q, n_head, n_head_kv, head_dim);
    if (rc || (rc = check_geometry(T_kv, n_head, n_head_kv, head_dim))) return rc;
    if ((rc = check_attn(scale, precision)) || (rc = check_window(window, causal))) return rc;
    if (precision == PFA_PREC_F32)
        return fail(PFA_ERR_INVALID_ARG, "qk_prep_chunk_attn_tiled takes PFA_PREC_BF16, "
                                         "PFA_PREC_BF16X3 or PFA_PREC_F16 (the f32 mode reads "
                                         "the f32 cache: qk_prep_chunk_attn)");
    if ((rc = check_rope(head_dim, rope_dim, rope_freq_base, rms_eps))) return rc;
    if (max_rows < 1) return fail(PFA_ERR_INVALID_ARG, "max_rows must be >= 1 (got %d)", max_rows);
    pfa::SeqTable st;
    if ((rc = build_chunk_seqs(q_offsets, kv_offsets, n_seqs, T_q, T_kv, st))) return rc;
    if (T_q == 0) return PFA_OK;
    if (!q_norm_w || !k_norm_w) return fail(PFA_ERR_INVALID_ARG, "null norm weights");
    pfa::PrepParams prep{q_norm_w, k_norm_w, nullptr, rope_dim, rms_eps, (double)rope_freq_base};
    const int cap_tiles = (max_rows + pfa::kBf16TileKeys - 1) / pfa::kBf16TileKeys;
    return attn_common(Mode::kChunkTiled, q, k, v, out, k_cache, v_cache, gate, gate_per_head,
                       st, n_head, n_head_kv, head_dim, scale, causal, window, precision, &prep,
                       workspace, workspace_bytes, stream, kv_tiles, cap_tiles);
}

// ---------------------------------------------------------------------------
// 8-bit quantised session (needle-core v3/model.rs: Q, K and V quantised per
// (token, head) after RoPE; attention through the int8 store).

// A device buffer an entry point reads or writes, for the overlap checks.
struct Span {
    const void* p;
    size_t n;
    bool written;
    const char* name;
};

// No written span may overlap another span (reads may alias each other).
static int check_spans(const Span* sp, int n) {
    for (int i = 0; i < n; ++i)
        for (int j = i + 1; j < n; ++j)
            if ((sp[i].written || sp[j].written) && sp[i].p && sp[j].p &&
                overlaps(sp[i].p, sp[i].n, sp[j].p, sp[j].n))
                return fail(PFA_ERR_INVALID_ARG, "%s must not overlap %s", sp[i].name, sp[j].name);
    return PFA_OK;
}

// Workspace of the 8-bit attention: the K/V tiles and the tiles' key scales,
// then (fused entry) the Q codes and Q scales, then the key split's partial results.
struct Q8Layout {
    size_t scales_off = 0, qc_off = 0, qs_off = 0, part_off = 0, need = 0;
};
static Q8Layout q8_layout(const Plan& p, int T_q, int n_head, int head_dim, bool fused) {
    Q8Layout l;
    l.scales_off = pfa::q8_tile_bytes(p.sched.n_tiles, p.geom.Hkv, head_dim);
    size_t end = l.scales_off + pfa::q8_scale_bytes(p.sched.n_tiles, p.geom.Hkv);
    if (fused) {
        l.qc_off = align256(end);
        l.qs_off = align256(l.qc_off + (size_t)T_q * n_head * head_dim);
        end = l.qs_off + (size_t)T_q * n_head * 4;
    }
    l.part_off = p.part_bytes ? align256(end) : end;
    l.need = l.part_off + p.part_bytes;
    return l;
}

static int check_q8_attn(float scale) {
    if (!std::isfinite(scale) || !(scale > 0.0f))
        return fail(PFA_ERR_INVALID_ARG,
                    "the 8-bit entry points need a finite scale > 0 (got %g)", (double)scale);
    return PFA_OK;
}


size_t pfa_q8_workspace_bytes(const int32_t* q_offsets, const int32_t* kv_offsets, int n_seqs,
                              int T_q, int T_kv, int n_head, int n_head_kv, int head_dim,
                              int fused) {
    g_err[0] = 0;
    if (check_geometry(T_q, n_head, n_head_kv, head_dim) ||
        check_geometry(T_kv, n_head, n_head_kv, head_dim))
        return 0;
    if (T_q == 0) return 0;
    pfa::SeqTable st;
    if (build_chunk_seqs(q_offsets, kv_offsets, n_seqs, T_q, T_kv, st)) return 0;
    Plan p;
    if (make_plan(st, n_head, n_head_kv, head_dim, 1.0f, 1, PFA_PREC_BF16, p)) return 0;
    if (p.items == 0) return 0;
    return q8_layout(p, T_q, n_head, head_dim, fused != 0).need;
}

int pfa_quantize_rows(const float* x, int64_t n_rows, int row_len, int8_t* codes, float* scales,
                      float* x_fq, void* stream) {
    g_err[0] = 0;
    if (n_rows < 0) return fail(PFA_ERR_INVALID_ARG, "n_rows must be >= 0");
    if (row_len < 1 || row_len > (1 << 16))
        return fail(PFA_ERR_INVALID_ARG, "row_len must be in 1..65536 (got %d)", row_len);
    if (n_rows > (int64_t(1) << 40) / row_len)
        return fail(PFA_ERR_UNSUPPORTED, "n_rows * row_len exceeds 2^40");
    if (n_rows == 0) return PFA_OK;
    if (!x || !codes || !scales) return fail(PFA_ERR_INVALID_ARG, "null tensor pointer");
    const size_t n = (size_t)n_rows * row_len;
    // x_fq may be x itself (in place); otherwise no buffer may overlap another
    const Span sp[4] = {{x, n * 4, false, "x"},
                        {codes, n, true, "codes"},
                        {scales, (size_t)n_rows * 4, true, "scales"},
                        {x_fq == x ? nullptr : x_fq, n * 4, true, "x_fq"}};
    int rc = check_spans(sp, 4);
    if (rc) return rc;
    if (x_fq == x && (overlaps(x, n * 4, codes, n) || overlaps(x, n * 4, scales, n_rows * 4)))
        return fail(PFA_ERR_INVALID_ARG, "codes and scales must not overlap x");
    return hip_status(pfa::launch_quant_rows(x, n_rows, row_len, codes, scales, x_fq,
                                             (hipStream_t)stream),
                      "pfa_quantize_rows launch");
}

// Shared part of gqa_attn_q8 (store given) and qk_prep_attn_q8 (raw rows prepared,
// quantised and appended to the caller's store first).
static int attn_q8_common(bool fused, pfa::Q8Store in, const float* q, const float* k,
                          const float* v, float* out, const float* gate, int gate_per_head,
                          const pfa::SeqTable& st, int n_head, int n_head_kv, int head_dim,
                          float scale, int causal, int window, const pfa::PrepParams* prep,
                          void* workspace, size_t workspace_bytes, void* stream) {
    const int T_q = st.off[st.n_seqs], T_kv = st.koff[st.n_seqs];
    if (T_q == 0) return PFA_OK;
    if (!out || !in.k || !in.ks || !in.v || !in.vs || (!fused && (!in.q || !in.qs)) ||
        (fused && (!q || !k || !v)))
        return fail(PFA_ERR_INVALID_ARG, "null tensor pointer");
    if (!aligned16(in.k) || !aligned16(in.v) || (!fused && !aligned16(in.q)))
        return fail(PFA_ERR_INVALID_ARG, "8-bit code arrays must be 16-byte aligned");
    Plan p;
    int rc;
    if ((rc = make_plan(st, n_head, n_head_kv, head_dim, scale, causal, PFA_PREC_BF16, p)))
        return rc;
    if (p.items == 0) return PFA_OK;
    p.geom.window = window;
    p.geom.gate = gate;
    p.geom.gate_per_head = gate_per_head ? 1 : 0;
    const Q8Layout l = q8_layout(p, T_q, n_head, head_dim, fused);
    if (!workspace)
        return fail(PFA_ERR_INVALID_ARG, "the 8-bit attention needs a workspace (%zu bytes)",
                    l.need);
    if (workspace_bytes < l.need)
        return fail(PFA_ERR_INVALID_ARG, "workspace of %zu bytes, %zu needed", workspace_bytes,
                    l.need);
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
        return fail(PFA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    const size_t qrow = (size_t)T_q * n_head, krow = (size_t)T_kv * n_head_kv;
    const size_t newk = (size_t)T_q * n_head_kv * head_dim;
    const Span sp[12] = {
        {out, qrow * head_dim * 4, true, "out"},
        {gate, gate ? qrow * (gate_per_head ? 1 : head_dim) * 4 : 0, false, "gate"},
        {workspace, l.need, true, "the workspace"},
        {fused ? nullptr : in.q, qrow * head_dim, false, "q"},
        {fused ? nullptr : in.qs, qrow * 4, false, "q_scale"},
        {in.k, krow * head_dim, fused, "k_cache"},
        {in.ks, krow * 4, fused, "k_scale"},
        {in.v, krow * head_dim, fused, "v_cache"},
        {in.vs, krow * 4, fused, "v_scale"},
        {fused ? q : nullptr, qrow * head_dim * 4, false, "q"},
        {fused ? k : nullptr, newk * 4, false, "k"},
        {fused ? v : nullptr, newk * 4, false, "v"}};
    if ((rc = check_spans(sp, 12))) return rc;
    char* ws = static_cast<char*>(workspace);
    const pfa::Partials part = p.partials(ws + l.part_off);
    if ((rc = check_aligned({out, gate, q, k, v, prep ? prep->wq : nullptr,
                             prep ? prep->wk : nullptr})))
        return rc;
    const char* what = fused ? "qk_prep_attn_q8 launch" : "gqa_attn_q8 launch";
    if (fused) {
        // the new rows: Q and K normalised and rotated at their positions, then Q (into
        // the workspace), K and V (into the last rows of each sequence's store range)
        // quantised
        in.q = reinterpret_cast<int8_t*>(ws + l.qc_off);
        in.qs = reinterpret_cast<float*>(ws + l.qs_off);
        const pfa::Q8Rows rows{const_cast<int8_t*>(in.q), const_cast<float*>(in.qs),
                               const_cast<int8_t*>(in.k), const_cast<float*>(in.ks),
                               const_cast<int8_t*>(in.v), const_cast<float*>(in.vs)};
        if ((rc = hip_status(pfa::launch_qknorm_rope_q8(q, k, v, prep->wq, prep->wk, st, T_q,
                                                        n_head, n_head_kv, head_dim,
                                                        prep->rope_dim, (float)prep->base,
                                                        prep->eps, rows, (hipStream_t)stream),
                             what)))
            return rc;
    }
    return hip_status(pfa::launch_attn_q8(in, out, workspace, p.sched, p.geom, head_dim, part,
                                          p.items, (hipStream_t)stream),
                      what);
}

int gqa_attn_q8(const int8_t* q, const float* q_scale, const int8_t* k_cache,
                const float* k_scale, const int8_t* v_cache, const float* v_scale, float* out,
                const float* gate, int gate_per_head, const int32_t* q_offsets,
                const int32_t* kv_offsets, int n_seqs, int T_q, int T_kv, int n_head,
                int n_head_kv, int head_dim, float scale, int causal, int window,
                void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    int rc = check_geometry(T_q, n_head, n_head_kv, head_dim);
    if (rc || (rc = check_geometry(T_kv, n_head, n_head_kv, head_dim))) return rc;
    if ((rc = check_q8_attn(scale)) || (rc = check_window(window, causal))) return rc;
    pfa::SeqTable st;
    if ((rc = build_chunk_seqs(q_offsets, kv_offsets, n_seqs, T_q, T_kv, st))) return rc;
    if (T_q == 0) return PFA_OK;
    const pfa::Q8Store in{q, q_scale, k_cache, k_scale, v_cache, v_scale};
    return attn_q8_common(false, in, nullptr, nullptr, nullptr, out, gate, gate_per_head, st,
                          n_head, n_head_kv, head_dim, scale, causal, window, nullptr, workspace,
                          workspace_bytes, stream);
}

int qk_prep_attn_q8(const float* q, const float* k, const float* v, float* out,
                    const float* gate, int gate_per_head, const float* q_norm_w,
                    const float* k_norm_w, int8_t* k_cache, float* k_scale, int8_t* v_cache,
                    float* v_scale, const int32_t* q_offsets, const int32_t* kv_offsets,
                    int n_seqs, int T_q, int T_kv, int n_head, int n_head_kv, int head_dim,
                    int rope_dim, float rope_freq_base, float rms_eps, float scale, int causal,
                    int window, void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    int rc = check_geometry(T_q, n_head, n_head_kv, head_dim);
    if (rc || (rc = check_geometry(T_kv, n_head, n_head_kv, head_dim))) return rc;
    if ((rc = check_q8_attn(scale)) || (rc = check_window(window, causal))) return rc;
    if ((rc = check_rope(head_dim, rope_dim, rope_freq_base, rms_eps))) return rc;
    pfa::SeqTable st;
    if ((rc = build_chunk_seqs(q_offsets, kv_offsets, n_seqs, T_q, T_kv, st))) return rc;
    if (T_q == 0) return PFA_OK;
    if (!q_norm_w || !k_norm_w) return fail(PFA_ERR_INVALID_ARG, "null norm weights");
    pfa::PrepParams prep{q_norm_w, k_norm_w, nullptr, rope_dim, rms_eps, (double)rope_freq_base};
    const pfa::Q8Store in{nullptr, nullptr, k_cache, k_scale, v_cache, v_scale};
    return attn_q8_common(true, in, q, k, v, out, gate, gate_per_head, st, n_head, n_head_kv,
                          head_dim, scale, causal, window, &prep, workspace, workspace_bytes,
                          stream);
}

// ---------------------------------------------------------------------------
// Plan report: what an attention call would enqueue, decided by the same host code the
// entry points run (plan_call / make_plan), and the work unit every attention
// workgroup decodes (the kernels' own decode, compiled for the host too).

namespace {

// Rotary pairing of the QK-norm + RoPE kernel (its template argument): both halves of a
// pair in one lane (rope_dim = head_dim = 128), partner lane ^ 32 (rope_dim 64), general.
int qknorm_mode(int head_dim, int rope_dim) {
    if (head_dim == 128 && rope_dim == 128) return 0;
    return rope_dim == 64 ? 1 : 2;
}

void append(char* buf, size_t n, const char* fmt, ...) {
    const size_t used = strlen(buf);
    if (used + 1 >= n) return;
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf + used, n - used, fmt, ap);
    va_end(ap);
}

// Names of the kernels one call enqueues, in order (as the launchers instantiate them).
void kernel_names(int entry, int precision, int D, int rope_dim, const Plan& p, char* buf,
                  size_t n) {
    buf[0] = 0;
    const bool tiled = entry == PFA_ENTRY_CHUNK_TILED;
    const bool fused = entry == PFA_ENTRY_PREP || entry == PFA_ENTRY_CHUNK_PREP ||
                       entry == PFA_ENTRY_Q8_PREP || tiled;
    const bool split_keys = p.sched.max_chunks > 1;
    const char* merge = p.counters ? "true" : "false";  // split items merged in place
    const char* sep = "";
    if (entry == PFA_ENTRY_Q8 || entry == PFA_ENTRY_Q8_PREP) {
        if (fused) {
            append(buf, n, "qknorm_rope_kernel<%d,%d,true>", D, qknorm_mode(D, rope_dim));
            sep = " + ";
        }
        append(buf, n,
               "%sstage_kv_q8_kernel<%d,%s> + attn_bf16_kernel<%d,false,false,true,%s,false>",
               sep, D, D == 128 ? "true" : "false", D, merge);
    } else if (precision == PFA_PREC_F32) {
        if (fused) {
            append(buf, n, "qknorm_rope_kernel<%d,%d,false> + ", D, qknorm_mode(D, rope_dim));
        }
        append(buf, n, "attn_f32_kernel<%d,%s,%s,%s>", D, fused ? "true" : "false",
               p.sched.paired ? "true" : "false", merge);
    } else {
        const char* sp = precision == PFA_PREC_BF16X3 ? "true" : "false";
        const char* hf = precision == PFA_PREC_F16 ? "true" : "false";
        if (entry == PFA_ENTRY_CHUNK_PREP || tiled) {
            append(buf, n, "qknorm_rope_kernel<%d,%d,false> + ", D, qknorm_mode(D, rope_dim));
        }
        if (tiled) {
            append(buf, n,
                   "append_tiles_kernel<%d,%s,%s> + attn_bf16_kernel<%d,%s,true,false,%s,%s>", D,
                   sp, hf, D, sp, merge, hf);
            if (split_keys && !p.counters) append(buf, n, " + attn_combine_kernel<%d>", D);
            return;
        }
        if (fused) append(buf, n, "rope_table_kernel<%d,%s> + ", D, sp);
        append(buf, n,
               "stage_kv_bf16_kernel<%d,%s,%s,%s> + attn_bf16_kernel<%d,%s,%s,false,%s,%s>", D,
               sp, entry == PFA_ENTRY_PREP ? "true" : "false", hf, D, sp,
               fused ? "true" : "false", merge, hf);
    }
    if (split_keys && !p.counters) append(buf, n, " + attn_combine_kernel<%d>", D);
}

// Arguments of a plan query -> sequence table and plan (what the entry point would do).
int plan_query(int entry, const int32_t* q_offsets, const int32_t* kv_offsets, int n_seqs,
               int T_q, int T_kv, int n_head, int n_head_kv, int head_dim, int rope_dim,
               int causal, int window, int precision, int has_k_rot_out, size_t ws_bytes,
               CallPlan& cp, pfa::SeqTable& st, size_t& need) {
    int rc;
    if (entry < PFA_ENTRY_PREFILL || entry > PFA_ENTRY_CHUNK_TILED)
        return fail(PFA_ERR_INVALID_ARG, "unknown entry %d", entry);
    const bool tiled = entry == PFA_ENTRY_CHUNK_TILED;
    if (tiled && precision == PFA_PREC_F32)
        return fail(PFA_ERR_INVALID_ARG, "qk_prep_chunk_attn_tiled takes PFA_PREC_BF16, "
                                         "PFA_PREC_BF16X3 or PFA_PREC_F16");
    const bool prefill = entry == PFA_ENTRY_PREFILL || entry == PFA_ENTRY_PREP;
    const bool q8 = entry == PFA_ENTRY_Q8 || entry == PFA_ENTRY_Q8_PREP;
    const bool fused = entry == PFA_ENTRY_PREP || entry == PFA_ENTRY_CHUNK_PREP ||
                       entry == PFA_ENTRY_Q8_PREP || tiled;
    if (prefill) T_kv = T_q;
    if ((rc = check_geometry(T_q, n_head, n_head_kv, head_dim)) ||
        (rc = check_geometry(T_kv, n_head, n_head_kv, head_dim)))
        return rc;
    if (q8) precision = PFA_PREC_BF16;  // the 8-bit kernels run on the bf16 schedule
    if ((rc = check_attn(1.0f, precision))) return rc;
    if (!prefill && (rc = check_window(window, causal))) return rc;
    if (fused && (rc = check_rope(head_dim, rope_dim, 1e4f, 0.0f))) return rc;
    if (prefill) {
        if ((rc = build_seqs(q_offsets, n_seqs, T_q, st))) return rc;
        window = 0;
    } else if ((rc = build_chunk_seqs(q_offsets, kv_offsets, n_seqs, T_q, T_kv, st))) {
        return rc;
    }
    const Mode mode = q8                                  ? Mode::kChunk
                      : tiled                             ? Mode::kChunkTiled
                      : entry == PFA_ENTRY_PREFILL        ? Mode::kPlain
                      : entry == PFA_ENTRY_PREP           ? Mode::kFused
                      : entry == PFA_ENTRY_CHUNK          ? Mode::kChunk
                                                          : Mode::kChunkFused;
    if ((rc = plan_call(mode, st, n_head, n_head_kv, head_dim, 1.0f, causal, window, precision,
                        has_k_rot_out != 0, ws_bytes, cp)))
        return rc;
    need = q8 ? (cp.p.items ? q8_layout(cp.p, T_q, n_head, head_dim, fused).need : 0)
              : (cp.p.items ? cp.need : 0);
    return PFA_OK;
}

}  // namespace

int pfa_attn_plan(int entry, const int32_t* q_offsets, const int32_t* kv_offsets, int n_seqs,
                  int T_q, int T_kv, int n_head, int n_head_kv, int head_dim, int rope_dim,
                  int causal, int window, int precision, int has_k_rot_out,
                  size_t workspace_bytes, pfa_plan* plan) {
    g_err[0] = 0;
    if (!plan) return fail(PFA_ERR_INVALID_ARG, "null plan pointer");
    memset(plan, 0, sizeof(*plan));
    CallPlan cp;
    pfa::SeqTable st;
    size_t need = 0;
    int rc = plan_query(entry, q_offsets, kv_offsets, n_seqs, T_q, T_kv, n_head, n_head_kv,
                        head_dim, rope_dim, causal, window, precision, has_k_rot_out,
                        workspace_bytes, cp, st, need);
    if (rc) return rc;
    const Plan& p = cp.p;
    plan->items = p.items;
    plan->rows_per_item = p.sched.rows_per_item;
    plan->waves_per_workgroup = p.waves;
    plan->tile_keys = p.tile_keys;
    plan->key_chunk_tiles = p.sched.kchunk;
    plan->max_key_chunks = p.sched.max_chunks;
    plan->paired = p.sched.paired;
    plan->merge_in_place = p.counters ? 1 : 0;
    const long long slots =
        p.sched.paired ? (p.items + 1) / 2 : (long long)p.items * p.sched.max_chunks;
    plan->workgroups = p.items ? slots * p.geom.chunks * p.geom.Hkv : 0;
    plan->workspace_bytes = need;
    const bool q8 = entry == PFA_ENTRY_Q8 || entry == PFA_ENTRY_Q8_PREP;
    if (p.items)
        kernel_names(entry, q8 ? PFA_PREC_BF16 : precision, head_dim, rope_dim, p, plan->kernels,
                     sizeof(plan->kernels));
    return PFA_OK;
}

int64_t pfa_attn_units(int entry, const int32_t* q_offsets, const int32_t* kv_offsets,
                       int n_seqs, int T_q, int T_kv, int n_head, int n_head_kv, int head_dim,
                       int rope_dim, int causal, int window, int precision, int has_k_rot_out,
                       size_t workspace_bytes, int32_t* records, int64_t max_records) {
    g_err[0] = 0;
    if (max_records < 0 || (max_records > 0 && !records))
        return fail(PFA_ERR_INVALID_ARG, "records: null with max_records > 0");
    CallPlan cp;
    pfa::SeqTable st;
    size_t need = 0;
    int rc = plan_query(entry, q_offsets, kv_offsets, n_seqs, T_q, T_kv, n_head, n_head_kv,
                        head_dim, rope_dim, causal, window, precision, has_k_rot_out,
                        workspace_bytes, cp, st, need);
    if (rc) return rc;
    const Plan& p = cp.p;
    if (p.items == 0) return 0;
    const int hk = p.geom.chunks * p.geom.Hkv;
    const long long slots =
        p.sched.paired ? (p.items + 1) / 2 : (long long)p.items * p.sched.max_chunks;
    const long long n_wg = slots * hk;
    int64_t n_rec = 0;
    for (long long wg = 0; wg < n_wg; ++wg) {
        // the paired f32 kernel: slot j takes item j, then item n - 1 - j (see attn_f32.hip)
        int bids[2] = {(int)wg, -1};
        if (p.sched.paired) {
            const int j = (int)(wg / hk), j2 = p.items - 1 - j;
            if (j2 > j) bids[1] = j2 * hk + (int)(wg % hk);
        }
        for (int pass = 0; pass < 2 && bids[pass] >= 0; ++pass) {
            const pfa::WorkItem wi = pfa::decode_item(p.sched, p.geom, bids[pass]);
            const pfa::KeyRange kr = pfa::item_key_range(p.sched, p.geom, wi, p.tile_keys);
            if (n_rec < max_records) {
                int32_t* r = records + n_rec * PFA_UNIT_FIELDS;
                r[0] = (int32_t)wg;
                r[1] = pass;
                r[2] = wi.item;
                r[3] = wi.sid;
                r[4] = wi.sb;
                r[5] = wi.kc;
                r[6] = wi.kv;
                r[7] = wi.chunk;
                r[8] = kr.t_begin;
                r[9] = kr.t_end;
            }
            ++n_rec;
        }
    }
    return n_rec;
}

}  // extern "C"
