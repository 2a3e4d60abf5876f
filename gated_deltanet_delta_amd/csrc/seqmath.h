// seqmath.h -- index arithmetic of packed sequences, chunk slots and state pools.
//
// Host and device functions alike: the kernels call them, and a host build of the same header is
// unit-tested under AddressSanitizer and UndefinedBehaviorSanitizer against malformed offsets.  A
// cu_seqlens array that is not non-decreasing from 0 to T is a caller error; these helpers clamp it
// so that every token range they return lies inside [0, T] and every chunk slot inside the
// workspace: malformed offsets give wrong numbers, never an access outside the buffers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kChunk = 64;   // tokens per chunk of the chunked kernels

// Sequence n's token range [t0, t1) inside batch row `row`, clamped to 0 <= t0 <= t1 <= T.
__host__ __device__ inline void sequence_range(const int32_t* cu_seqlens, int n, int T, int& row, int& t0,
                                               int& t1) {
    if (cu_seqlens) {
        int a = cu_seqlens[n], b = cu_seqlens[n + 1];
        a = a < 0 ? 0 : (a > T ? T : a);
        b = b < a ? a : (b > T ? T : b);
        row = 0;
        t0 = a;
        t1 = b;
    } else {
        row = n;
        t0 = 0;
        t1 = T;
    }
}

// Number of 64-token chunks of sequence n (its last chunk may be partial).
__host__ __device__ inline int sequence_chunks(const int32_t* cu_seqlens, int n, int T) {
    int row, t0, t1;
    sequence_range(cu_seqlens, n, T, row, t0, t1);
    const int len = t1 - t0;
    return len / kChunk + (len % kChunk != 0);
}

// State slot of sequence (or batch row) n: n itself, or state_indices[n] in a pool of num_slots
// states.  An index outside [0, num_slots) marks a padding row, which has no state: false is
// returned and slot is set to 0 (any in-bounds value; nothing is read or written through it).
__host__ __device__ inline bool state_slot(const int32_t* state_indices, int num_slots, int n, int& slot) {
    if (!state_indices) {
        slot = n;
        return true;
    }
    const int s = state_indices[n];
    const bool ok = s >= 0 && s < num_slots;
    slot = ok ? s : 0;
    return ok;
}

// Chunk slot -> (sequence n, chunk index ci, batch row, first token t0, length len).
struct ChunkLoc {
    int n, ci, row, t0, len;
};

// Locate chunk slot `slot`.  Packed input (cu_seqlens set): chunk_start[n] is the number of chunks of
// sequences 0..n-1 (sequence_chunks summed), chunk_start[N] the total; the slot belongs to the
// sequence whose chunk range holds it (zero-length sequences own none).  Otherwise every batch row
// has nct = ceil(T / 64) chunks.  Returns false for a slot past the last chunk; on true,
// 0 <= t0 < t0 + len <= T and 1 <= len <= 64.
__host__ __device__ inline bool locate_chunk(int slot, const int32_t* cu_seqlens, const int32_t* chunk_start,
                                             int N, int T, int nct, ChunkLoc& loc) {
    if (cu_seqlens) {
        if (slot < 0 || slot >= chunk_start[N]) return false;
        int lo = 0, hi = N;  // largest n with chunk_start[n] <= slot
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (chunk_start[mid] <= slot) lo = mid; else hi = mid;
        }
        // skip zero-length sequences that share the same start
        int n = lo;
        while (n + 1 < N && chunk_start[n + 1] <= slot) ++n;
        int row, a, b;
        sequence_range(cu_seqlens, n, T, row, a, b);
        loc.n = n;
        loc.ci = slot - chunk_start[n];
        loc.row = row;
        loc.t0 = a + loc.ci * kChunk;
        loc.len = b - loc.t0 < kChunk ? b - loc.t0 : kChunk;
        return loc.len > 0;
    }
    if (slot < 0 || nct <= 0) return false;
    loc.n = slot / nct;
    loc.ci = slot % nct;
    loc.row = loc.n;
    loc.t0 = loc.ci * kChunk;
    loc.len = T - loc.t0 < kChunk ? T - loc.t0 : kChunk;
    return loc.len > 0;
}

}  // namespace gdn
