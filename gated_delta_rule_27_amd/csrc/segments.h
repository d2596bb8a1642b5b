// segments.h — splitting each head's chunks into segments run by separate
// workgroups, for chunk kernels whose grid would leave compute units idle.
//
// The state entering a chunk depends only on the chunks before it ("Linear
// Attention, Visualized", "Chunkwise algorithm": "Update the state"), so a
// workgroup that owns chunks [c_s, c_{s+1}) first forms that state in a
// state-only pass over chunks [0, c_s) (no outputs), then runs its own chunks
// as usual.  Such a prefix chunk costs a fraction a of a full chunk step, so
// segment lengths shrink by the factor 1 - a from one to the next and every
// workgroup finishes at about the same time.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <cstdlib>

namespace linattn {

constexpr int kMaxSeg = 4;

// a compile-time integer as a value (a tag for generic lambdas)
template <int N>
struct IntC {
    static constexpr int value = N;
};

// segment s covers chunks [c[s], c[s+1]); n = 1 is the whole sequence
struct SegSplit {
    int n;
    int c[kMaxSeg + 1];
};

// The split for nchunks chunks and nblocks workgroups of one segment each:
// as many segments (at most kMaxSeg, at least four chunks each) as the compute
// units hold beside the unsplit grid.  Every segment reads s0 and only the last
// writes s_final, so a state updated in place (the two ranges of state_bytes
// overlapping) keeps one segment.  LINATTN_SEGMENTS=n (1..4) fixes the count.
inline SegSplit seg_split(int64_t nchunks, int64_t nblocks, bool allow, const void* s0, const void* s_final,
                          size_t state_bytes, double prefix_cost)
{
    SegSplit sp{};
    sp.n = 1;
    sp.c[0] = 0;
    sp.c[1] = (int)nchunks;
    if (!allow || nchunks < 2 || nblocks <= 0) return sp;
    if (s0 && s_final) {
        const char* a0 = static_cast<const char*>(s0);
        const char* a1 = static_cast<const char*>(s_final);
        if (a0 < a1 + state_bytes && a1 < a0 + state_bytes) return sp;
    }
    int64_t n = 0;
    if (const char* e = getenv("LINATTN_SEGMENTS")) {
        n = atoi(e);
        if (n < 1 || n > kMaxSeg) n = 0;
    }
    if (n == 0) {
        int dev = 0, ncu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
            return sp;
        n = ncu / nblocks;
        if (n > kMaxSeg) n = kMaxSeg;
        if (n > nchunks / 4) n = nchunks / 4;
    }
    if (n > nchunks) n = nchunks;
    if (n < 2) return sp;
    double w[kMaxSeg], tot = 0.0, f = 1.0;
    for (int i = 0; i < n; ++i, f *= 1.0 - prefix_cost) tot += (w[i] = f);
    sp.n = (int)n;
    double acc = 0.0;
    for (int i = 0; i < n; ++i) {
        acc += w[i];
        int64_t c = i + 1 == n ? nchunks : (int64_t)(nchunks * acc / tot + 0.5);
        if (c < sp.c[i] + 1) c = sp.c[i] + 1;
        if (c > nchunks - (n - 1 - i)) c = nchunks - (n - 1 - i);
        sp.c[i + 1] = (int)c;
    }
    return sp;
}

}  // namespace linattn
