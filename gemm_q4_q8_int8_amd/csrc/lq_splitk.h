// Device side of the GEMV split-K hand-off (single- and multi-token GEMV):
// the workgroups of one 64-row tile each sum a K slice, publish it to the
// caller's workspace, and the last one to arrive adds the slices in slice
// order.  Not installed.
//
// Memory ordering on gfx950.  Partial sums are written with relaxed
// agent-scope atomic stores and read with relaxed agent-scope atomic loads:
// both bypass the per-XCD L2 (which is not coherent between XCDs) and are
// performed at the device's coherence point.  A wave's vector memory counter
// only drops once such a store is acknowledged there, so a wave that waits
// for it (s_waitcnt 0) before its arrival RMW has made its partials visible
// device-wide before the counter moves; the last arrival issues its loads
// only after its RMW has returned.  Agent-scope release / acquire fences
// would give the same order by writing back and invalidating a whole L2 per
// workgroup, which made split launches several times slower.
#pragma once

#include "lq_internal.h"

namespace lq {

// Arrival of one K slice at its tile's counter; true for the last of S.  A
// counter word is (tag << 16) | arrivals.  Every launch has a tag of its own
// (next_splitk_tag), so a word holding anything else (zero, another launch's
// count, bytes an unrelated call left in the workspace) counts as no
// arrival yet: the workspace needs no clearing.  The last arrival clears
// the word, so a captured graph, which replays one tag, finds it clear on
// every replay.
//
// The first arrival claims the word with one compare-and-swap (from zero,
// or from whatever else it holds); every later one finds the tag there and
// counts itself with one fetch-add: the word keeps this launch's tag until
// the last arrival clears it, which cannot happen before this arrival.  So
// an arrival costs at most two atomics however many slices meet (a
// compare-and-swap retried until it wins costs O(S^2) atomics per tile when
// the S slices arrive together).  The claim loop ends: only an arrival of
// this launch moves a word away from a foreign value, and after it the word
// holds the tag.
__device__ __forceinline__ bool splitk_arrive(uint64_t* cnt, uint64_t tag, int S) {
    const uint64_t base = tag << 16;
    uint64_t cur = 0;   // the usual state of a word before its first arrival
    uint64_t n = 1;
    while (!__hip_atomic_compare_exchange_strong(cnt, &cur, base + 1, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT)) {
        if ((cur & ~uint64_t(0xFFFF)) == base) {
            n = (__hip_atomic_fetch_add(cnt, uint64_t(1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 0xFFFF) + 1;
            break;
        }
    }
    const bool last = n == uint64_t(S);
    if (last) __hip_atomic_store(cnt, uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return last;
}

// Store of one partial sum (see the ordering note above).
__device__ __forceinline__ void splitk_put(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until this wave's partial-sum stores are performed device-wide; the
// signal fences keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void splitk_publish() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// sum_{j < S} p[j * pitch] in slice order, loads issued eight at a time so
// their latencies overlap.
__device__ __forceinline__ float sum_slices(const float* p, size_t pitch, int S) {
    float t = 0.0f;
    for (int j = 0; j < S; j += 8) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float* q = p + size_t(min(j + k, S - 1)) * pitch;
            v[k] = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (j + k < S) t += v[k];
    }
    return t;
}

}  // namespace lq
