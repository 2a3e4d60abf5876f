// host_checks.cpp -- host build of libgdn's index arithmetic and argument checks, run under
// AddressSanitizer and UndefinedBehaviorSanitizer (test infrastructure).
//
// Part 1: the packed-sequence helpers the kernels use (seqmath.h) on malformed cu_seqlens arrays
// (decreasing, negative, past T, extreme values): every token range stays inside [0, T], every chunk
// slot the workspace layout reserves maps to tokens inside [0, T] or to nothing, and the scan's
// per-sequence chunk count (clamped to the workspace) never reaches past it.
// Part 2: the C entry points with rejected arguments return an error status without touching memory,
// and the workspace-size queries survive extreme sizes.
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "gdn.h"
#include "seqmath.h"

static int failures = 0;
#define CHECK(cond, ...)                                          \
    do {                                                          \
        if (!(cond)) {                                            \
            ++failures;                                           \
            std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            std::fprintf(stderr, __VA_ARGS__);                    \
            std::fprintf(stderr, "\n");                           \
        }                                                         \
    } while (0)

static void check_offsets(const std::vector<int32_t>& cu, int T, const char* what) {
    const int N = (int)cu.size() - 1;
    std::vector<int32_t> start(N + 1, 0);
    for (int n = 0; n < N; ++n) {
        int row, t0, t1;
        gdn::sequence_range(cu.data(), n, T, row, t0, t1);
        CHECK(row == 0 && 0 <= t0 && t0 <= t1 && t1 <= T, "%s: sequence %d range [%d, %d)", what, n, t0, t1);
        const int c = gdn::sequence_chunks(cu.data(), n, T);
        CHECK(c >= 0 && (long long)c * gdn::kChunk < (long long)T + gdn::kChunk, "%s: %d chunks", what, c);
        CHECK(start[n] <= INT_MAX - c, "%s: chunk count overflow", what);
        start[n + 1] = start[n] + c;
    }
    // the workspace reserves floor(T / 64) + N chunk slots for a packed call; probe past both ends
    const int slots = T / gdn::kChunk + N;
    const int last = (start[N] > slots ? start[N] : slots) + 3;
    const int stride = last > 100000 ? last / 50000 : 1;   // long cases: both ends plus a stride
    for (int slot = -2; slot < last; slot += (slot > 1000 && slot < last - 1000) ? stride : 1) {
        gdn::ChunkLoc loc{};
        if (!gdn::locate_chunk(slot, cu.data(), start.data(), N, T, 0, loc)) continue;
        CHECK(loc.n >= 0 && loc.n < N, "%s: slot %d -> sequence %d", what, slot, loc.n);
        CHECK(loc.t0 >= 0 && loc.len >= 1 && loc.len <= gdn::kChunk && loc.t0 + loc.len <= T,
              "%s: slot %d -> tokens [%d, %d)", what, slot, loc.t0, loc.t0 + loc.len);
    }
    // the scan walks min(chunks, slots - start[n]) chunks from slot start[n]: all inside the workspace
    for (int n = 0; n < N; ++n) {
        const int c = gdn::sequence_chunks(cu.data(), n, T);
        const int room = slots - start[n] > 0 ? slots - start[n] : 0;
        const int walked = c < room ? c : room;
        CHECK(walked == 0 || start[n] + walked <= slots, "%s: sequence %d walks past the workspace", what, n);
    }
}

static void part1() {
    const int T = 1000;
    check_offsets({0, 100, 400, 1000}, T, "valid");
    check_offsets({0, 0, 0, 1000}, T, "empty sequences");
    check_offsets({0, 500, 200, 1000}, T, "decreasing");
    check_offsets({-50, 100, -7, 1000}, T, "negative");
    check_offsets({0, 2000, 3000, 5000}, T, "past T");
    check_offsets({INT_MIN, INT_MAX, INT_MIN, INT_MAX}, T, "extremes");
    check_offsets({0, 1000, 0, 1000, 0, 1000}, T, "overlapping whole ranges");
    check_offsets({1000, 0}, T, "reversed single");
    check_offsets({0, 0}, 0, "no tokens");
    check_offsets({0, 5, INT_MAX - 3}, INT_MAX - 3, "lengths near the int range");
    // unpacked: every batch row has ceil(T / 64) chunks
    for (int slot = -1; slot < 3 * 16 + 2; ++slot) {
        gdn::ChunkLoc loc{};
        if (!gdn::locate_chunk(slot, nullptr, nullptr, 3, T, 16, loc)) continue;
        CHECK(loc.t0 >= 0 && loc.t0 + loc.len <= T && loc.row == slot / 16, "unpacked slot %d", slot);
    }
    gdn::ChunkLoc loc{};
    CHECK(!gdn::locate_chunk(0, nullptr, nullptr, 1, 0, 0, loc), "T = 0 has no chunks");
    // state pools: an index outside [0, num_slots) is a padding row with slot 0
    const int32_t idx[] = {3, -1, 4, INT_MIN, INT_MAX, 0};
    for (int n = 0; n < 6; ++n) {
        int slot = -99;
        const bool ok = gdn::state_slot(idx, 4, n, slot);
        CHECK(ok == (idx[n] >= 0 && idx[n] < 4), "state_slot %d", n);
        CHECK(slot >= 0 && slot < 4, "state_slot %d -> %d", n, slot);
    }
}

static void part2() {
    // fake, aligned, never dereferenced device addresses: every call below is rejected on the host
    void* p = reinterpret_cast<void*>(uintptr_t(1) << 20);
    float* f = static_cast<float*>(p);
    const int32_t* cu = static_cast<const int32_t*>(p);
    const gdn_dtype bf = GDN_BF16;
    CHECK(gdn_chunk_fwd(p, p, p, p, p, f, nullptr, 1, 64, 3, 4, 128, 128, 1, bf, bf, f, f, p, 1 << 30, nullptr)
              == GDN_ERROR_INVALID_VALUE, "Hv %% Hk != 0");
    CHECK(gdn_chunk_fwd(p, p, p, p, p, f, cu, 2, 64, 2, 4, 128, 128, 1, bf, bf, f, f, p, 1 << 30, nullptr)
              == GDN_ERROR_INVALID_VALUE, "cu_seqlens with B != 1");
    CHECK(gdn_chunk_fwd(p, p, p, p, p, f, nullptr, 1, -1, 2, 4, 128, 128, 1, bf, bf, f, f, p, 1 << 30, nullptr)
              == GDN_ERROR_INVALID_VALUE, "T < 0");
    CHECK(gdn_chunk_fwd(p, p, p, p, p, f, nullptr, 1, 64, 2, 4, 96, 128, 1, bf, bf, f, f, p, 1 << 30, nullptr)
              == GDN_ERROR_NOT_SUPPORTED, "dk = 96");
    CHECK(gdn_chunk_fwd(p, p, p, p, p, f, nullptr, 1, 64, 2, 4, 128, 128, 1, bf, bf, f, f, nullptr, 0, nullptr)
              == GDN_ERROR_WORKSPACE, "missing workspace");
    CHECK(gdn_chunk_fwd(p, p, p, p, p, f, nullptr, INT_MAX, INT_MAX, 2, 4, 128, 128, INT_MAX, bf, bf, f, f, p,
                        1 << 30, nullptr) == GDN_ERROR_INVALID_VALUE, "sizes that overflow");
    CHECK(gdn_chunk_fwd(p, p, p, p, p, f, nullptr, 1, 64, 2, 4, 128, 128, 1, (gdn_dtype)7, bf, f, f, p, 1 << 30,
                        nullptr) == GDN_ERROR_INVALID_VALUE, "bad dtype");
    CHECK(gdn_recurrent_step(p, p, p, p, p, f, 1, 0, 2, 4, 128, 128, bf, bf, f, nullptr) == GDN_ERROR_INVALID_VALUE,
          "decode with T = 0");
    CHECK(gdn_recurrent_step(p, p, p, p, p, reinterpret_cast<float*>(uintptr_t(1) << 20 | 4), 1, 1, 2, 4, 128, 128,
                             bf, bf, f, nullptr) == GDN_ERROR_INVALID_VALUE, "misaligned state");
    CHECK(gdn_chunk_bwd(p, p, p, p, p, f, nullptr, f, f, 1, 64, 2, 4, 128, 128, 1, bf, bf, f, f, f, f, f, f, p, 0,
                        nullptr) == GDN_ERROR_WORKSPACE, "backward without workspace");
    CHECK(gdn_gated_rmsnorm(f, p, f, -1.f, 10, 128, bf, bf, p, nullptr) == GDN_ERROR_INVALID_VALUE, "eps < 0");
    CHECK(gdn_causal_conv1d(p, f, nullptr, p, nullptr, 0, nullptr, 1, 10, 64, 17, 1, bf, 1, p, nullptr)
              == GDN_ERROR_NOT_SUPPORTED, "conv width 17");
    const int ext[] = {INT_MIN, -1, 0, 1, 64, INT_MAX};
    for (int B : ext)
        for (int T : ext)
            for (int N : ext) {
                (void)gdn_chunk_fwd_workspace_size(B, T, 16, 32, 128, 128, N, bf);
                (void)gdn_chunk_bwd_workspace_size(B, T, 16, 32, 128, 128, N);
                (void)gdn_chunk_bwd_ex_workspace_size(B, T, 16, 32, 128, 128, N, bf, 1, 1, GDN_FLAG_QK_L2NORM);
            }
    CHECK(gdn_chunk_fwd_workspace_size(1, 4096, 16, 32, 128, 128, 1, bf) > 0, "workspace of the prefill");
    CHECK(gdn_chunk_fwd_workspace_size(INT_MAX, INT_MAX, 16, 32, 128, 128, INT_MAX, bf) == 0, "oversized query");
}

int main() {
    part1();
    part2();
    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("host checks passed\n");
    return 0;
}
