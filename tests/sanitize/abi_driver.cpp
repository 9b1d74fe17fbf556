// abi_driver.cpp -- exercises libpfa's host code (argument checks, sequence tables, work
// schedules, workspace layouts, the plan report) under AddressSanitizer and UBSan.
//
// Every call here is either a size / plan query or one the library must reject before
// anything is enqueued (bad pointers, shapes, tables, workspaces), so the driver never
// launches a kernel and needs no GPU.  Host arrays are heap-allocated at their exact
// sizes, so a read or write one element past them is reported.  Exit status 0 when every
// check holds; a sanitizer report aborts the process.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "pfa.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what) {
    if (!ok) {
        std::fprintf(stderr, "FAILED: %s (last error: %s)\n", what, pfa_last_error());
        ++failures;
    }
}

// Rejected with a non-OK status and a message.
void rejected(int status, const char* what) {
    expect(status != PFA_OK && std::strlen(pfa_last_error()) > 0, what);
}

uint64_t rng_state = 0x9E3779B97F4A7C15ull;
uint32_t rnd(uint32_t n) {  // xorshift64*, uniform enough for table shapes
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 33) % n;
}

// An exactly-sized heap copy of cumulative offsets of `lens`.
int32_t* offsets(const std::vector<int>& lens) {
    int32_t* o = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * (lens.size() + 1)));
    o[0] = 0;
    for (size_t i = 0; i < lens.size(); ++i) o[i + 1] = o[i] + lens[i];
    return o;
}

void* fake(uintptr_t mib) { return reinterpret_cast<void*>(mib << 20); }  // never dereferenced

void argument_checks() {
    float* f = static_cast<float*>(fake(1));
    float* o = static_cast<float*>(fake(64));
    // geometry and flags
    rejected(gqa_prefill_attn(f, f, f, o, nullptr, 0, 16, 4, 2, 96, 0.125f, 1, 0, nullptr, 0,
                              nullptr), "head_dim 96");
    rejected(gqa_prefill_attn(f, f, f, o, nullptr, 0, 16, 5, 2, 64, 0.125f, 1, 0, nullptr, 0,
                              nullptr), "n_head not a multiple");
    rejected(gqa_prefill_attn(f, f, f, o, nullptr, 0, 16, 4, 2, 64, 0.125f, 1, 7, nullptr, 0,
                              nullptr), "bad precision");
    rejected(gqa_prefill_attn(nullptr, f, f, o, nullptr, 0, 16, 4, 2, 64, 0.125f, 1, 0, nullptr,
                              0, nullptr), "null q");
    rejected(gqa_prefill_attn(f, f, f, f, nullptr, 0, 16, 4, 2, 64, 0.125f, 1, 0, nullptr, 0,
                              nullptr), "out aliases q");
    rejected(gqa_prefill_attn(f, f, f, o, nullptr, 0, 16, 4, 2, 64, 0.125f, 1, PFA_PREC_BF16,
                              nullptr, 0, nullptr), "bf16 without workspace");
    // sequence tables
    std::vector<int> lens = {5, 0, 11};
    int32_t* offs = offsets(lens);
    rejected(gqa_prefill_attn(f, f, f, o, offs, 3, 15, 4, 2, 64, 0.125f, 1, 0, nullptr, 0,
                              nullptr), "offsets end != T");
    offs[2] = 3;  // decreasing
    rejected(gqa_prefill_attn(f, f, f, o, offs, 3, 16, 4, 2, 64, 0.125f, 1, 0, nullptr, 0,
                              nullptr), "decreasing offsets");
    std::free(offs);
    std::vector<int> many(PFA_MAX_SEQS + 1, 1);
    offs = offsets(many);
    rejected(gqa_prefill_attn(f, f, f, o, offs, PFA_MAX_SEQS + 1, PFA_MAX_SEQS + 1, 4, 2, 64,
                              0.125f, 1, 0, nullptr, 0, nullptr), "too many sequences");
    std::free(offs);
    // rope and norm arguments
    rejected(qknorm_rope(f, f, o, o, f, f, nullptr, 0, 16, 4, 2, 64, 63, 1e4f, 1e-6f, nullptr),
             "odd rope_dim");
    rejected(qknorm_rope(f, f, o, o, f, f, nullptr, 0, 16, 4, 2, 64, 64, -1.0f, 1e-6f, nullptr),
             "negative base");
    rejected(qk_prep_attn(f, f, f, o, nullptr, f, nullptr, 0, 16, 4, 2, 64, 64, 1e4f, 1e-6f,
                          0.125f, 1, 0, nullptr, nullptr, 0, nullptr), "null norm weights");
    // chunk entries: caches shorter than their queries, offsets in pairs, windows
    std::vector<int> ql = {4, 4}, kl = {8, 3};
    int32_t* qo = offsets(ql);
    int32_t* ko = offsets(kl);
    rejected(gqa_chunk_attn(f, f, f, o, nullptr, 0, qo, ko, 2, 8, 11, 4, 2, 64, 0.125f, 1, 0, 0,
                            nullptr, 0, nullptr), "cache shorter than queries");
    rejected(gqa_chunk_attn(f, f, f, o, nullptr, 0, qo, nullptr, 2, 8, 11, 4, 2, 64, 0.125f, 1,
                            0, 0, nullptr, 0, nullptr), "one offset table");
    rejected(gqa_chunk_attn(f, f, f, o, nullptr, 0, nullptr, nullptr, 0, 8, 8, 4, 2, 64, 0.125f,
                            0, 16, 0, nullptr, 0, nullptr), "window without causal");
    std::free(qo);
    std::free(ko);
    // 8-bit entries
    int8_t* c8 = static_cast<int8_t*>(fake(3));
    rejected(gqa_attn_q8(c8, f, c8, f, c8, f, o, nullptr, 0, nullptr, nullptr, 0, 8, 8, 4, 2, 64,
                         0.0f, 1, 0, nullptr, 0, nullptr), "q8 scale 0");
    rejected(pfa_quantize_rows(f, 10, 0, c8, f, nullptr, nullptr), "row_len 0");
    // misaligned tensors
    float* mis = reinterpret_cast<float*>(reinterpret_cast<char*>(f) + 4);
    rejected(gqa_prefill_attn(mis, f, f, o, nullptr, 0, 16, 4, 2, 64, 0.125f, 1, 0, nullptr, 0,
                              nullptr), "misaligned q");
    // T = 0 is a no-op without pointers
    expect(gqa_prefill_attn(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0, 4, 2, 64, 0.125f,
                            1, 0, nullptr, 0, nullptr) == PFA_OK, "T = 0");
}

void random_tables(int rounds) {
    const int geoms[][3] = {{8, 8, 128}, {16, 8, 128}, {32, 8, 128}, {16, 4, 64}, {6, 2, 128},
                            {8, 1, 64}};
    for (int r = 0; r < rounds; ++r) {
        const int n = 1 + (int)rnd(PFA_MAX_SEQS);
        std::vector<int> ql(n), kl(n);
        for (int s = 0; s < n; ++s) {
            ql[s] = rnd(8) == 0 ? 0 : (int)rnd(r % 3 == 0 ? 2000 : 300);
            kl[s] = ql[s] + (r % 2 ? (int)rnd(3000) : 0);
        }
        int32_t* qo = offsets(ql);
        int32_t* ko = offsets(kl);
        const int T_q = qo[n], T_kv = ko[n];
        const int* g = geoms[rnd(6)];
        const int H = g[0], Hkv = g[1], D = g[2];
        for (int prec = 0; prec < 3; ++prec) {
            (void)pfa_workspace_bytes(qo, n, T_q, H, Hkv, D, prec, (int)rnd(2));
            (void)pfa_chunk_workspace_bytes(qo, ko, n, T_q, T_kv, H, Hkv, D, prec, (int)rnd(2));
        }
        (void)pfa_q8_workspace_bytes(qo, ko, n, T_q, T_kv, H, Hkv, D, (int)rnd(2));
        for (int entry = PFA_ENTRY_PREFILL; entry <= PFA_ENTRY_Q8_PREP; ++entry) {
            const bool prefill = entry <= PFA_ENTRY_PREP;
            const int prec = (int)rnd(3), window = prefill ? 0 : (int)rnd(3) * 100;
            const size_t ws = rnd(4) == 0 ? 0 : SIZE_MAX;
            pfa_plan* plan = static_cast<pfa_plan*>(std::malloc(sizeof(pfa_plan)));
            const int rc = pfa_attn_plan(entry, qo, prefill ? nullptr : ko, n, T_q, T_kv, H, Hkv,
                                         D, D, 1, window, prec, (int)rnd(2), ws, plan);
            expect(rc == PFA_OK, "plan of a valid table");
            const int64_t cnt = pfa_attn_units(entry, qo, prefill ? nullptr : ko, n, T_q, T_kv,
                                               H, Hkv, D, D, 1, window, prec, 0, ws, nullptr, 0);
            expect(cnt >= 0, "unit count");
            if (cnt > 0) {
                int32_t* rec = static_cast<int32_t*>(
                    std::malloc(sizeof(int32_t) * PFA_UNIT_FIELDS * (size_t)cnt));
                const int64_t got = pfa_attn_units(entry, qo, prefill ? nullptr : ko, n, T_q,
                                                   T_kv, H, Hkv, D, D, 1, window, prec, 0, ws,
                                                   rec, cnt);
                expect(got == cnt, "unit records");
                // a shorter buffer: exactly max_records written, the full count returned
                const int64_t part = pfa_attn_units(entry, qo, prefill ? nullptr : ko, n, T_q,
                                                    T_kv, H, Hkv, D, D, 1, window, prec, 0, ws,
                                                    rec, cnt / 2);
                expect(part == cnt, "unit count with a short buffer");
                std::free(rec);
            }
            std::free(plan);
        }
        std::free(qo);
        std::free(ko);
    }
}

}  // namespace

int main() {
    std::printf("%s\n", pfa_version());
    argument_checks();
    random_tables(300);
    std::printf("abi driver: %d failures\n", failures);
    return failures ? 1 : 0;
}
