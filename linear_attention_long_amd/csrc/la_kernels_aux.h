// la_kernels_aux.h -- chunk planner, chunk-state prefix scan, output gate,
// decode step and state fill.
#pragma once

#include "la_device.h"
#include "la_items.h"

namespace la {

// Chunk table of a packed batch: chunk_off[s] = first item of sequence s,
// chunk_off[nseq] = number of items, with chunks of C tokens.  With
// search != 0 the kernel first picks C on the device: the smallest multiple
// of 64 in [c_lo, C] with sum_s ceil(L_s / C) <= max_items (a binary search;
// the count does not increase with C, and C itself must qualify), stored in
// chunk_off[nseq + 1].  One workgroup of 256 threads.
__device__ __forceinline__ int32_t block_sum_256(int32_t v, int32_t* red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    const int tid = threadIdx.x;
    __syncthreads();  // red is free
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(256) void k_plan_chunks(const int32_t* __restrict__ cu, int32_t nseq,
                                                     int32_t C, int32_t* __restrict__ chunk_off,
                                                     int32_t search, int32_t c_lo,
                                                     int32_t max_items) {
    __shared__ int32_t part[257];
    __shared__ int32_t red[4];
    const int tid = threadIdx.x;
    const int per = (nseq + 255) / 256;
    const int s0 = min(nseq, tid * per), s1 = min(nseq, s0 + per);
    if (search) {
        int32_t lo = max(1, c_lo / 64), hi = C / 64;  // C (= 64 * hi) qualifies
        while (lo < hi) {
            const int32_t mid = (lo + hi) >> 1, cm = 64 * mid;
            int32_t local = 0;
            for (int s = s0; s < s1; ++s) local += (max(0, cu[s + 1] - cu[s]) + cm - 1) / cm;
            if (block_sum_256(local, red) <= max_items) hi = mid; else lo = mid + 1;
        }
        C = 64 * hi;
        if (tid == 0) chunk_off[nseq + 1] = C;
    }
    int32_t local = 0;
    for (int s = s0; s < s1; ++s) {
        const int32_t L = max(0, cu[s + 1] - cu[s]);
        local += (L + C - 1) / C;
    }
    part[tid] = local;
    __syncthreads();
    if (tid == 0) {
        int32_t acc = 0;
        for (int i = 0; i < 256; ++i) {
            const int32_t x = part[i];
            part[i] = acc;
            acc += x;
        }
        part[256] = acc;
        chunk_off[nseq] = acc;
    }
    __syncthreads();
    int32_t acc = part[tid];
    for (int s = s0; s < s1; ++s) {
        chunk_off[s] = acc;
        const int32_t L = max(0, cu[s + 1] - cu[s]);
        acc += (L + C - 1) / C;
    }
}

// Exclusive prefix over the chunks of each sequence, in increasing chunk order
// (deterministic): buf[item] <- init + sum of the earlier chunks' increments.
// The main pass writes each sequence's final state after its last chunk;
// here only sequences without tokens get theirs (= init).  E = D*D (+ D with
// the normaliser).
__global__ __launch_bounds__(256) void k_chunk_scan(float* __restrict__ buf, int64_t stride,
                                                    ItemMap map, int H, int D, int E,
                                                    const float* state_in, const float* z_in,
                                                    float* state_out, float* z_out,
                                                    uint64_t* __restrict__ xclear, int64_t nclear,
                                                    const float* __restrict__ half, int32_t cps2) {
    // the fused gate's exchange buffer (when the main pass that follows has
    // one) is cleared here too, which saves a launch
    if (xclear) {
        const int64_t nthr = (int64_t)gridDim.x * gridDim.y * gridDim.z * 256;
        const int64_t gid =
            (((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * 256 + threadIdx.x;
        for (int64_t i = gid; i < nclear; i += nthr) xclear[i] = 0ull;
    }
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= E) return;
    const int h = blockIdx.y, s = blockIdx.z;
    int32_t first, count;
    seq_items(map, s, first, count);
    const int32_t row = state_row(map, s);
    const int DD = D * D;
    float acc = 0.f;
    if (row >= 0) {
        if (e < DD) acc = state_in ? state_in[((size_t)row * H + h) * DD + e] : 0.f;
        else acc = z_in ? z_in[((size_t)row * H + h) * D + (e - DD)] : 0.f;
    }
    // eight increments in flight at a time, then their prefixes in order (the
    // last chunk has no increment: the main pass writes the final state).
    // With `half` (equal-length sequences) chunk i's increment is the sum of
    // the increments of its half chunks 2i and 2i + 1, held there.
    constexpr int U = 8;
    const size_t h0 = (size_t)s * cps2;
    for (int32_t i0 = 0; i0 < count; i0 += U) {
        float dlt[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int32_t i = i0 + j;
            dlt[j] = 0.f;
            if (i < count - 1)
                dlt[j] = half ? half[((h0 + 2 * i) * H + h) * stride + e] +
                                    half[((h0 + 2 * i + 1) * H + h) * stride + e]
                              : buf[((size_t)(first + i) * H + h) * stride + e];
        }
#pragma unroll
        for (int j = 0; j < U; ++j) {
            if (i0 + j < count) buf[((size_t)(first + i0 + j) * H + h) * stride + e] = acc;
            acc += dlt[j];
        }
    }
    // a sequence with no tokens has no main-pass item: its final state is its
    // initial one
    if (row < 0 || count > 0) return;
    if (e < DD) {
        if (state_out) state_out[((size_t)row * H + h) * DD + e] = acc;
    } else if (z_out) {
        z_out[((size_t)row * H + h) * D + (e - DD)] = acc;
    }
}

// n 64-bit words <- 0 (clears the fused gate's exchange buffer; a plain
// kernel rather than a memset node so the call stays graph-capturable).
__global__ __launch_bounds__(256) void k_zero_u64(uint64_t* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0ull;
}

// For every (sequence, head) = blockIdx.y: state_out row <- state_in row (or
// zeros), z likewise -- the state of sequences the main pass does not write
// (no tokens).  Rows follow the map's slot table; an in-place array (the same
// pointer in and out) is left as it is.
__global__ __launch_bounds__(256) void k_fill_state(const float* state_in, const float* z_in,
                                                    float* state_out, float* z_out, ItemMap map,
                                                    int H, int D) {
    const int s = blockIdx.y / H, h = blockIdx.y - (blockIdx.y / H) * H;
    const int32_t row = state_row(map, s);
    if (row < 0) return;
    const int DD = D * D;
    const size_t sb = ((size_t)row * H + h) * DD, zb = ((size_t)row * H + h) * D;
    for (int e = blockIdx.x * 256 + threadIdx.x; e < DD + D; e += gridDim.x * 256) {
        if (e < DD) {
            if (state_out && state_out != state_in) state_out[sb + e] = state_in ? state_in[sb + e] : 0.f;
        } else if (z_out && z_out != z_in) {
            z_out[zb + e - DD] = z_in ? z_in[zb + e - DD] : 0.f;
        }
    }
}

// Output gate (page "MiniMax-Text-01 405B MoE模型架构与训练策略解析" section 2.1):
// per token and norm group of G features, r = 1/sqrt(mean(y^2) + eps), then
// out = y * r * w * sigmoid(x).  One wave per (token, group); y and out may be
// the same buffer.
template <typename XT, typename OutT>
__global__ __launch_bounds__(256) void k_gate(const float* y, const XT* __restrict__ x,
                                              const float* __restrict__ w, OutT* out, int64_t ntok,
                                              int F, int G, float eps) {
    const int lane = threadIdx.x & 63;
    const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int ngroups = F / G;
    const int64_t tok = unit / ngroups;
    if (tok >= ntok) return;
    const int grp = (int)(unit - tok * ngroups);
    const size_t base = (size_t)tok * F + (size_t)grp * G;
    float ss = 0.f;
    for (int f = lane; f < G; f += 64) {
        const float a = y[base + f];
        ss += a * a;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    const float r = 1.0f / sqrtf(ss / (float)G + eps);
    for (int f = lane; f < G; f += 64) {
        const float a = y[base + f];
        const float wf = w ? w[grp * G + f] : 1.f;
        store_from_f32<OutT>(out + base + f, a * r * wf * sigmoid(load_as_f32<XT>(x + base + f)));
    }
}

template <typename XT> struct Vec4In;
template <> struct Vec4In<float> {
    static __device__ __forceinline__ void load(const float* p, float (&v)[4]) {
        const float4 t = *(const float4*)p;
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    }
};
template <> struct Vec4In<uint16_t> {
    static __device__ __forceinline__ void load(const uint16_t* p, float (&v)[4]) {
        const uint2 t = *(const uint2*)p;
        v[0] = bf16_lo_to_f32(t.x); v[1] = bf16_hi_to_f32(t.x);
        v[2] = bf16_lo_to_f32(t.y); v[3] = bf16_hi_to_f32(t.y);
    }
};
template <typename OutT> __device__ __forceinline__ void store_vec4(OutT* p, const float (&v)[4]);
template <> __device__ __forceinline__ void store_vec4<float>(float* p, const float (&v)[4]) {
    *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
}
template <> __device__ __forceinline__ void store_vec4<uint16_t>(uint16_t* p, const float (&v)[4]) {
    *(uint2*)p = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

// Gate for groups of G = 256 * NC features: one wave per (token, group), each
// lane holds 4 * NC features in registers between the sum of squares and the
// scaling, and issues all of its loads before using any of them.
template <typename XT, typename OutT, int NC>
__global__ __launch_bounds__(256) void k_gate4(const float* y, const XT* __restrict__ x,
                                               const float* __restrict__ w, OutT* out, int64_t ntok,
                                               int F, int G, float eps) {
    const int lane = threadIdx.x & 63;
    const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int ngroups = F / G;
    const int64_t tok = unit / ngroups;
    if (tok >= ntok) return;
    const int grp = (int)(unit - tok * ngroups);
    const size_t base = (size_t)tok * F + (size_t)grp * G + 4 * lane;
    float yv[NC][4], xv[NC][4];
#pragma unroll
    for (int j = 0; j < NC; ++j) Vec4In<float>::load(y + base + 256 * j, yv[j]);
#pragma unroll
    for (int j = 0; j < NC; ++j) Vec4In<XT>::load(x + base + 256 * j, xv[j]);
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) ss += yv[j][e] * yv[j][e];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    const float r = 1.0f / sqrtf(ss / (float)G + eps);
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        float wv[4] = {1.f, 1.f, 1.f, 1.f};
        if (w) Vec4In<float>::load(w + (size_t)grp * G + 4 * lane + 256 * j, wv);
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = yv[j][e] * r * wv[e] * sigmoid(xv[j][e]);
        store_vec4<OutT>(out + base + 256 * j, o);
    }
}

// Decode step (page "六十四：MiniMax-01" section 3: a new token updates only S
// and z, and reads its output from them).  One workgroup per (sequence,
// head) streams the d x d state once: S += phi(k) phi(v)^T in place, then
// y = phi(q)^T S (read after the update), optionally / phi(q).z.
// With a slot table (slots != nullptr) the state of sequence n is row
// slots[n] of S and z (rows of them); a slot outside [0, rows) gives y = 0
// and touches no state.
// STREAM: the state is read and written with non-temporal hints (it is not
// kept in the caches); with SPLIT = 1 each workgroup then streams its
// (sequence, head)'s d x d block contiguously.  That is the faster form when
// the state is not cache-resident between calls (measured on MI355X: 92 us
// against 105 us per step for 64 x 64 heads of d = 128 whose state was last
// touched 768 MiB of traffic earlier); when it is resident, SPLIT = 4 without
// hints is faster (70 against 91 us).
template <int D, typename InT, typename OutT, bool NORM, int SPLIT, bool STREAM = false>
__global__ __launch_bounds__(256) void k_decode(const InT* __restrict__ q, const InT* __restrict__ k,
                                                const InT* __restrict__ v, float* __restrict__ S,
                                                float* __restrict__ z, OutT* __restrict__ y,
                                                const int32_t* __restrict__ slots, int32_t rows,
                                                int H, int feat) {
    // SPLIT workgroups per (sequence, head), each owning D / SPLIT value
    // columns of the state (more, smaller workgroups stream better); the
    // normaliser is shared by all columns, so the normalised mode is unsplit
    static_assert(!NORM || SPLIT == 1, "the normalised mode updates z in one workgroup");
    constexpr int DC = D / SPLIT;  // value columns of this workgroup
    constexpr int CQ = DC / 4;     // threads per state row (float4 each)
    constexpr int RG = 256 / CQ;   // row groups
    constexpr int M = D / RG;      // rows per thread
    __shared__ float fq[D], fk[D], fv[DC];
    __shared__ float4 part[RG][CQ];
    __shared__ float dpart[4];
    const int tid = threadIdx.x;
    const size_t pair = blockIdx.x / SPLIT;  // sequence * H + head (token rows)
    const int c0 = (int)(blockIdx.x % SPLIT) * DC;
    const size_t vb = pair * D;
    size_t spair = pair;             // row * H + head (state rows)
    if (slots) {
        const int n = (int)(pair / H), h = (int)(pair - (size_t)n * H);
        const int32_t r = slots[n];
        if (r < 0 || r >= rows) {
            if (tid < DC) store_from_f32<OutT>(y + vb + c0 + tid, 0.f);
            return;
        }
        spair = (size_t)r * H + h;
    }
    // feat: the inputs are feature vectors already (no SiLU here)
    if (tid < D) {
        const float xq = load_as_f32<InT>(q + vb + tid), xk = load_as_f32<InT>(k + vb + tid);
        fq[tid] = feat ? xq : silu(xq);
        fk[tid] = feat ? xk : silu(xk);
    }
    if (tid < DC) {
        const float xv = load_as_f32<InT>(v + vb + c0 + tid);
        fv[tid] = feat ? xv : silu(xv);
    }
    __syncthreads();
    float den_part = 0.f;
    if (NORM && tid < D) {
        const float zn = z[spair * D + tid] + fk[tid];
        z[spair * D + tid] = zn;
        den_part = fq[tid] * zn;
    }
    const int cq = tid % CQ, rg = tid / CQ;
    const f32x4_t v4 = {fv[4 * cq], fv[4 * cq + 1], fv[4 * cq + 2], fv[4 * cq + 3]};
    f32x4_t* S4 = (f32x4_t*)(S + spair * D * D + c0);
    f32x4_t s[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const f32x4_t* p = S4 + (rg + RG * m) * (D / 4) + cq;
        s[m] = STREAM ? __builtin_nontemporal_load(p) : *p;
    }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int i = rg + RG * m;
        const float kk = fk[i], qq = fq[i];
        const f32x4_t t = s[m] + kk * v4;
        f32x4_t* p = S4 + i * (D / 4) + cq;
        if (STREAM) __builtin_nontemporal_store(t, p);
        else *p = t;
        acc += qq * t;
    }
    part[rg][cq] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    if (NORM) {
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) den_part += __shfl_xor(den_part, m, 64);
        if ((tid & 63) == 0) dpart[tid >> 6] = den_part;
    }
    __syncthreads();
    if (tid < DC) {
        const int c4 = tid >> 2, e = tid & 3;
        float a = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            const float4 p = part[r][c4];
            a += e == 0 ? p.x : e == 1 ? p.y : e == 2 ? p.z : p.w;
        }
        if (NORM) a /= (dpart[0] + dpart[1] + dpart[2] + dpart[3]);
        store_from_f32<OutT>(y + vb + c0 + tid, a);
    }
}

}  // namespace la
