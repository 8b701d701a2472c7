// la_items.h -- mapping of a flat work-item index to (sequence, chunk).
//
// A sequence of L tokens is cut into ceil(L / C) chunks of C tokens (the
// last one shorter).  Each (chunk, head) pair is one workgroup; chunks of a
// sequence are independent once their starting state is known (a prefix sum
// of per-chunk state increments), which is an exact reassociation of the
// recurrent sum S_t = S_{t-1} + phi(k_t) phi(v_t)^T.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

struct ItemMap {
    const int32_t* cu;         // device [nseq+1] token offsets, or nullptr (equal lengths T)
    const int32_t* chunk_off;  // device [nseq+1] first item of each sequence (varlen only)
    int32_t nseq;
    int32_t T;                 // equal-length batches: tokens per sequence
    int32_t C;                 // tokens per chunk (multiple of 64)
    int32_t cps;               // equal-length batches: chunks per sequence
    int32_t cdev;              // varlen: 1 = the chunk length is chunk_off[nseq + 1]
                               // (chosen on the device), 0 = C
    const int32_t* slots;      // device [nseq] state rows, or nullptr (row = sequence)
    int32_t rows;              // rows of the state arrays when slots is given
};

// Row of sequence s in the state arrays: s itself, or slots[s] when a slot
// table is given; -1 for a slot outside [0, rows) (that sequence then starts
// from a zero state and writes none).
__device__ __forceinline__ int32_t state_row(const ItemMap& m, int32_t s) {
    if (!m.slots) return s;
    const int32_t r = m.slots[s];
    return (r >= 0 && r < m.rows) ? r : -1;
}

struct Item {
    int32_t seq;
    int32_t chunk;   // index within the sequence
    int64_t t0;      // first global token of the chunk
    int32_t len;     // tokens in the chunk (>= 1)
    bool last;       // last chunk of its sequence
    int32_t row;     // state row of the sequence (state_row), -1 for none
};

// Returns false for items past the end (the grid is sized by an upper bound).
__device__ __forceinline__ bool decode_item(const ItemMap& m, int32_t item, Item& it) {
    if (m.cu == nullptr) {
        if (item >= m.nseq * m.cps) return false;
        it.seq = item / m.cps;
        it.chunk = item - it.seq * m.cps;
        const int32_t start = it.chunk * m.C;
        it.t0 = (int64_t)it.seq * m.T + start;
        it.len = min(m.C, m.T - start);
        it.last = (it.chunk == m.cps - 1);
        it.row = state_row(m, it.seq);
        return it.len > 0;
    }
    if (item >= m.chunk_off[m.nseq]) return false;
    // last s with chunk_off[s] <= item (empty sequences have equal neighbours)
    int32_t lo = 0, hi = m.nseq;  // invariant: chunk_off[lo] <= item < chunk_off[hi]
    while (hi - lo > 1) {
        const int32_t mid = (lo + hi) >> 1;
        if (m.chunk_off[mid] <= item) lo = mid; else hi = mid;
    }
    it.seq = lo;
    it.chunk = item - m.chunk_off[lo];
    const int32_t C = m.cdev ? m.chunk_off[m.nseq + 1] : m.C;
    const int32_t s0 = m.cu[lo], s1 = m.cu[lo + 1];
    it.t0 = (int64_t)s0 + (int64_t)it.chunk * C;
    it.len = (int32_t)min((int64_t)C, (int64_t)s1 - it.t0);
    it.last = (it.chunk == m.chunk_off[lo + 1] - m.chunk_off[lo] - 1);
    it.row = state_row(m, it.seq);
    return it.len > 0;
}

// First item of a sequence and its item count.
__device__ __forceinline__ void seq_items(const ItemMap& m, int32_t s, int32_t& first, int32_t& count) {
    if (m.cu == nullptr) {
        first = s * m.cps;
        count = m.cps;
    } else {
        first = m.chunk_off[s];
        count = m.chunk_off[s + 1] - first;
    }
}

}  // namespace la
