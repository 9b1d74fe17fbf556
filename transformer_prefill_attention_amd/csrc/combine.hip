// combine.hip -- merges the partial results of attention items whose key range
// was split across workgroups (short inputs, see AttnSched::kchunk).
//
// The softmax of a row over the union of disjoint key chunks follows from each
// chunk's (m_k, l_k, O_k / l_k): with M = max_k m_k and w_k = l_k 2^(m_k - M)
// (m in log2 units, as the attention kernels keep it),
//   O = sum_k w_k (O_k / l_k) / sum_k w_k,
// the same rescaling the online softmax applies between tiles (memra-engine
// 0.130.0 src/forward.rs, SDPA block, for what is computed).  A chunk that saw
// no key of a row has l_k = 0 and weight 0.
#include "pfa_device.h"
#include "pfa_internal.h"

namespace pfa {

namespace {

constexpr int kThreads = 256;

// One workgroup per (item, head chunk, K/V head, wavefront of the attention
// workgroup): its 32 rows x D.  Eight threads per row, D/8 columns each; every
// thread reads its row's per-chunk (m, l) itself (eight-fold, from cache) so no
// synchronisation is needed.
template <int D>
__global__ __launch_bounds__(kThreads) void attn_combine_kernel(Partials part,
                                                                 float* __restrict__ out,
                                                                 AttnSched sched, AttnGeom geom,
                                                                 int waves, int tile_keys) {
    WorkItem w;
    int bid = blockIdx.x;
    const int wave = bid % waves;
    bid /= waves;
    w.kv = bid % geom.Hkv;
    bid /= geom.Hkv;
    w.chunk = bid % geom.chunks;
    w.item = bid / geom.chunks;
    w.kc = 0;
    decode_seq(sched, w);
    const int s1 = w.s1, q0 = w.q0;
    // the item's key chunks, counted as the attention kernel counts them
    const int n_chunks = item_key_range(sched, geom, w, tile_keys).n_chunks;
    if (n_chunks < 2) return;  // written directly by its only workgroup
    const int hloc = wave % geom.hpw, rblk = wave / geom.hpw;
    const int r = threadIdx.x >> 3, c0 = (threadIdx.x & 7) * (D / 8);
    const int row = q0 + rblk * 32 + r;
    if (row >= s1) return;
    const int h = w.kv * geom.g + w.chunk * geom.hpw + hloc;
    // slot of key chunk k: ((item * max_chunks + k) * chunks + chunk) * Hkv + kv units,
    // times the waves of a unit, plus this wavefront
    const size_t slot0 =
        (((size_t)w.item * sched.max_chunks * geom.chunks + w.chunk) * geom.Hkv + w.kv) * waves +
        wave;
    const size_t kstride = (size_t)geom.chunks * geom.Hkv * waves;  // slots between key chunks
    // One pass over the chunks, kBatch at a time: each batch's (m, l) and partial rows are
    // loaded together (up to kBatch chunks cost one memory round trip), and the running
    // merge is rescaled when a batch raises the running max -- the online softmax's own
    // rescaling, applied to whole chunks.
    constexpr int kBatch = 8;
    float m_run = -INFINITY, den = 0.0f;
    floatx4 acc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < n_chunks; k0 += kBatch) {
        float2 ml[kBatch];
        floatx4 o[kBatch][D / 32];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            // chunks past the count re-read the last one (always a written slot), weight 0
            const size_t slot = slot0 + (size_t)min(k0 + j, n_chunks - 1) * kstride;
            ml[j] = part.ml[slot * 32 + r];
            const float* src = part.o + (slot * 32 + r) * D + c0;
#pragma unroll
            for (int i = 0; i < D / 32; ++i) o[j][i] = *reinterpret_cast<const floatx4*>(src + 4 * i);
        }
        // a chunk that saw no key of the row has l = 0 and weight 0
        float mb = -INFINITY;
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            if (k0 + j < n_chunks && ml[j].y > 0.0f) mb = fmaxf(mb, ml[j].x);
        if (mb > m_run) {
            const float a = m_run == -INFINITY ? 0.0f : exp2f(m_run - mb);
            den *= a;
#pragma unroll
            for (int i = 0; i < D / 32; ++i) acc[i] *= a;
            m_run = mb;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const float wk = k0 + j < n_chunks && ml[j].y > 0.0f ? ml[j].y * exp2f(ml[j].x - m_run)
                                                                  : 0.0f;
            den += wk;
#pragma unroll
            for (int i = 0; i < D / 32; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][e] += wk * o[j][i][e];
        }
    }
    const float inv = 1.0f / den;
    float* dst = out + ((int64_t)row * geom.H + h) * D + c0;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
        floatx4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[i][e] * inv;
        if (geom.gate)
            x *= gate_factors(geom.gate, geom.gate_per_head, row, geom.H, h, D,
                              c0 + 4 * i);
        *reinterpret_cast<floatx4*>(dst + 4 * i) = x;
    }
}

}  // namespace

hipError_t launch_attn_combine(const Partials& part, float* out, const AttnSched& sched,
                               const AttnGeom& geom, int D, int waves, int tile_keys, int n_items,
                               hipStream_t stream) {
    const dim3 grid((unsigned)n_items * geom.chunks * geom.Hkv * waves), block(kThreads);
    if (D == 128)
        hipLaunchKernelGGL((attn_combine_kernel<128>), grid, block, 0, stream, part, out, sched,
                           geom, waves, tile_keys);
    else
        hipLaunchKernelGGL((attn_combine_kernel<64>), grid, block, 0, stream, part, out, sched,
                           geom, waves, tile_keys);
    return hipGetLastError();
}

}  // namespace pfa
