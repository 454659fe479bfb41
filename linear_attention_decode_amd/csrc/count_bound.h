// count_bound.h -- host-side bounds on a layer's ring counts.
//
// The handle keeps, from the calls that move the pointers, a range [lo, hi]
// holding count = pos - base of every sequence, and an upper bound on pos.
// A flush whose threshold no sequence can reach is then not launched at all:
// in the standard decode schedule (flush when the buffer is full, page
// "ReplaySSM: Cachear Inputs, No Estado", section "Como funciona en la
// practica") every sequence holds the same count, the range is exact, and
// that is every step but one in L.  The range only ever widens where a
// call's outcome depends on device data: a rollback (its amounts live on the
// device) drops lo to 0, and a call that may leave a sequence unchanged
// (ring overflow, pointer overflow) keeps that sequence's old count inside
// the range.  Plain C++, no device code.
#pragma once
#include <cstdint>

namespace replay {

struct CountBound {
    static constexpr int64_t kPosMax = 2147483647;   // pointers are int32
    int32_t L = 1;
    int32_t lo = 0, hi = 0;   // lo <= pos - base <= hi for every sequence; 0 <= lo <= hi <= L
    int64_t pos = 0;          // >= pos of every sequence

    static int32_t need(int32_t threshold) { return threshold > 1 ? threshold : 1; }
    static int32_t min2(int32_t a, int32_t b) { return a < b ? a : b; }

    void reset(int32_t ring_len) {
        L = ring_len;
        lo = hi = 0;
        pos = 0;
    }
    // a launch whose outcome is unknown (it failed): assume nothing
    void unknown() {
        lo = 0;
        hi = L;
        pos = kPosMax;
    }
    // checkpoint load: base = pos everywhere
    void load() { lo = hi = 0; }
    // rebuilt from every sequence's pointers as read back from the device:
    // the smallest and largest count and the largest pos.  Pointers outside
    // 0 <= base <= pos with count <= L leave the bounds as they were (false).
    bool from_pointers(const int32_t *pos_b, const int32_t *base_b, int32_t B) {
        int32_t l = L, h = 0;
        int64_t p = 0;
        for (int32_t b = 0; b < B; ++b) {
            const int64_t c = (int64_t)pos_b[b] - base_b[b];
            if (base_b[b] < 0 || c < 0 || c > L) return false;
            if (c < l) l = (int32_t)c;
            if (c > h) h = (int32_t)c;
            if (pos_b[b] > p) p = pos_b[b];
        }
        if (B < 1) l = 0;
        lo = l;
        hi = h;
        pos = p;
        return true;
    }
    // rollback: counts drop by amounts only the device knows
    void rollback() { lo = 0; }

    // append(W): needs count + W <= L and pos + W <= kPosMax, else the
    // sequence is left unchanged
    void append(int32_t W) {
        const bool reject = hi + W > L || pos + W > kPosMax;
        if (!reject) lo += W;
        hi = min2(hi + W, L);
        pos += W;
    }

    // flush(m): sequences with count >= max(m, 1) fold (count 0)
    bool flush_may_fold(int32_t min_count) const { return hi >= need(min_count); }
    void flush(int32_t min_count) {
        const int32_t n = need(min_count);
        if (lo >= n)
            lo = hi = 0;   // every sequence folds
        else if (hi >= n) {
            lo = 0;        // some fold, the rest stay below n
            hi = n - 1;
        }
    }

    // fused step: append one token; where the ring then holds >= max(f, 1)
    // entries, fold (count 0).  A sequence with count + 1 > L or pos at
    // kPosMax is left unchanged.
    void step(int32_t flush_at) {
        const int32_t n = need(flush_at);
        const bool reject = hi + 1 > L || pos >= kPosMax;
        if (reject) {
            // accepted sequences: 0, or below n and at most L; rejected ones
            // keep their count
            const int32_t h = min2(min2(hi + 1, L), n - 1);
            hi = hi > h ? hi : h;
            lo = 0;
        } else if (lo + 1 >= n) {
            lo = hi = 0;
        } else if (hi + 1 < n) {
            lo += 1;
            hi += 1;
        } else {
            lo = 0;
            hi = n - 1;
        }
        pos += 1;
    }

    // fused verify round: fold where count >= max(f, 1), then append W
    // drafts; a sequence whose drafts do not fit after that (or whose pointer
    // would pass kPosMax) is left unchanged
    void verify_round(int32_t flush_at, int32_t W) {
        const int32_t n = need(flush_at);
        const int32_t keep = hi < n ? hi : n - 1;     // >= every kept count (folded ones: 0)
        const int32_t keep_lo = lo >= n ? 0 : (hi >= n ? 0 : lo);
        const bool reject = keep + W > L || pos + W > kPosMax;
        const int32_t h = keep + W <= L ? keep + W : L;
        hi = reject && hi > h ? hi : h;
        lo = reject ? 0 : keep_lo + W;
        pos += W;
    }
};

}  // namespace replay
