// la_kernels_valu.h -- fp32 vector-ALU kernels: the exact-fp32 path.
//
// Used for fp32 inputs (fp32 arithmetic throughout), for head dim 64, and for
// block sizes other than the matrix-core kernel's 64.  Same method as the
// matrix-core kernels (page "MiniMax-Text-01 405B MoE模型架构与训练策略解析"
// section 2.1; page "六十四：MiniMax-01" section 3), evaluated with the block
// size B chosen by the caller: for each block, every query row takes
// phi(q) S_blockstart plus the masked quadratic form over the block's keys up
// to itself; then S += phi(K)^T phi(V) over the block.  Work is staged in
// 32-row sub-tiles, so any B that is a multiple of 32 keeps the same
// association as the blocked form.
#pragma once

#include "la_device.h"
#include "la_items.h"

namespace la {
namespace vk {

constexpr int NT = 256;
constexpr int SUB = 32;

template <int D>
struct SmemMain {
    float S[D * D];       // state at the start of the current block
    float fq[SUB * D];
    float fk[SUB * D];
    float fv[SUB * D];
    float P[SUB * (SUB + 1)];
    float z[D];
};

template <int D>
struct SmemState {
    float fk[SUB * D];
    float fv[SUB * D];
};

// phi of rows [0, nvalid) of a 32-row sub-tile of one head into LDS (fp32);
// rows past nvalid are zero.  feat: the inputs are features already (no SiLU).
template <int D, typename InT>
__device__ __forceinline__ void load_sub(float* dst, const InT* __restrict__ src, int64_t t0,
                                         int nvalid, int H, int h, int tid, int feat) {
    for (int e = tid; e < SUB * D; e += NT) {
        const int r = e / D, col = e % D;
        float x = 0.f;
        if (r < nvalid) {
            x = load_as_f32<InT>(src + ((size_t)(t0 + r) * H + h) * D + col);
            if (!feat) x = silu(x);
        }
        dst[e] = x;
    }
}

template <int D, typename InT, bool NORM>
__global__ __launch_bounds__(NT, 1) void k_valu_state(const InT* __restrict__ k,
                                                      const InT* __restrict__ v, ItemMap map, int H,
                                                      float* __restrict__ buf, int64_t buf_stride,
                                                      int feat) {
    constexpr int PER = D * D / NT;
    __shared__ SmemState<D> sm;
    const int tid = threadIdx.x, h = blockIdx.y;
    Item it;
    // (the last chunk of a sequence: the main pass writes the final state)
    if (!decode_item(map, blockIdx.x, it) || it.last) return;
    const int dv = tid % D, dk0 = tid / D;
    constexpr int DKS = NT / D;
    float s[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) s[m] = 0.f;
    float zacc = 0.f;
    for (int r0 = 0; r0 < it.len; r0 += SUB) {
        const int n = min(SUB, it.len - r0);
        __syncthreads();
        load_sub<D, InT>(sm.fk, k, it.t0 + r0, n, H, h, tid, feat);
        load_sub<D, InT>(sm.fv, v, it.t0 + r0, n, H, h, tid, feat);
        __syncthreads();
#pragma unroll 2
        for (int r = 0; r < SUB; ++r) {
            const float fvr = sm.fv[r * D + dv];
#pragma unroll
            for (int m = 0; m < PER; ++m) s[m] += sm.fk[r * D + dk0 + DKS * m] * fvr;
        }
        if (NORM && tid < D) {
            float a = 0.f;
            for (int r = 0; r < SUB; ++r) a += sm.fk[r * D + tid];
            zacc += a;
        }
    }
    float* dst = buf + ((size_t)blockIdx.x * H + h) * buf_stride;
#pragma unroll
    for (int m = 0; m < PER; ++m) dst[(dk0 + DKS * m) * D + dv] = s[m];
    if (NORM && tid < D) dst[D * D + tid] = zacc;
}

template <int D, typename InT, typename OutT, bool NORM>
__global__ __launch_bounds__(NT, 1) void k_valu_main(
    const InT* __restrict__ q, const InT* __restrict__ k, const InT* __restrict__ v, ItemMap map,
    int H, int B, const float* __restrict__ prefix, int64_t prefix_stride,
    const float* __restrict__ state_in, const float* __restrict__ z_in, OutT* __restrict__ y,
    float* state_out, float* z_out, int feat) {
    constexpr int CPT = D / 8;          // output columns per thread
    constexpr int PER = D * D / NT;     // state elements per thread
    constexpr int DKS = NT / D;
    __shared__ SmemMain<D> sm;
    const int tid = threadIdx.x, h = blockIdx.y;
    Item it;
    if (!decode_item(map, blockIdx.x, it)) return;

    const float* s0 = nullptr;
    const float* z0 = nullptr;
    if (prefix) {
        s0 = prefix + ((size_t)blockIdx.x * H + h) * prefix_stride;
        z0 = s0 + D * D;
    } else {
        if (state_in && it.row >= 0) s0 = state_in + ((size_t)it.row * H + h) * D * D;
        if (z_in && it.row >= 0) z0 = z_in + ((size_t)it.row * H + h) * D;
    }
    for (int e = tid; e < D * D; e += NT) sm.S[e] = s0 ? s0[e] : 0.f;
    if (NORM && tid < D) sm.z[tid] = z0 ? z0[tid] : 0.f;

    const int r = tid >> 3, cl = tid & 7;  // output row and column phase
    const int dv = tid % D, dk0 = tid / D;

    for (int b0 = 0; b0 < it.len; b0 += B) {
        const int blen = min(B, it.len - b0);
        const int nsub = (blen + SUB - 1) / SUB;
        for (int i = 0; i < nsub; ++i) {
            const int64_t tq = it.t0 + b0 + i * SUB;
            const int nq = min(SUB, blen - i * SUB);
            __syncthreads();
            load_sub<D, InT>(sm.fq, q, tq, nq, H, h, tid, feat);
            __syncthreads();
            float acc[CPT];
#pragma unroll
            for (int j = 0; j < CPT; ++j) acc[j] = 0.f;
            float den = 0.f;
            // inter-block: phi(q) . S_blockstart
            for (int dk = 0; dk < D; ++dk) {
                const float a = sm.fq[r * D + dk];
#pragma unroll
                for (int j = 0; j < CPT; ++j) acc[j] += a * sm.S[dk * D + cl + 8 * j];
                if (NORM) den += a * sm.z[dk];
            }
            // intra-block: masked quadratic form over the block's keys <= query
            for (int jj = 0; jj <= i; ++jj) {
                const int64_t tk = it.t0 + b0 + jj * SUB;
                const int nk = min(SUB, blen - jj * SUB);
                __syncthreads();
                load_sub<D, InT>(sm.fk, k, tk, nk, H, h, tid, feat);
                load_sub<D, InT>(sm.fv, v, tk, nk, H, h, tid, feat);
                __syncthreads();
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int cc = cl + 8 * m;
                    float p = 0.f;
                    if (jj < i || cc <= r)
                        for (int dk = 0; dk < D; ++dk) p += sm.fq[r * D + dk] * sm.fk[cc * D + dk];
                    sm.P[r * (SUB + 1) + cc] = p;
                }
                __syncthreads();
                for (int cc = 0; cc < SUB; ++cc) {
                    const float p = sm.P[r * (SUB + 1) + cc];
#pragma unroll
                    for (int j = 0; j < CPT; ++j) acc[j] += p * sm.fv[cc * D + cl + 8 * j];
                    if (NORM) den += p;
                }
            }
            if (r < nq) {
                const float sc = NORM ? 1.f / den : 1.f;
                OutT* dst = y + ((size_t)(tq + r) * H + h) * D;
#pragma unroll
                for (int j = 0; j < CPT; ++j) store_from_f32<OutT>(dst + cl + 8 * j, acc[j] * sc);
            }
        }
        // state update over the block's keys
        for (int jj = 0; jj < nsub; ++jj) {
            const int64_t tk = it.t0 + b0 + jj * SUB;
            const int nk = min(SUB, blen - jj * SUB);
            __syncthreads();
            load_sub<D, InT>(sm.fk, k, tk, nk, H, h, tid, feat);
            load_sub<D, InT>(sm.fv, v, tk, nk, H, h, tid, feat);
            __syncthreads();
            float a[PER];
#pragma unroll
            for (int m = 0; m < PER; ++m) a[m] = 0.f;
#pragma unroll 2
            for (int rr = 0; rr < SUB; ++rr) {
                const float fvr = sm.fv[rr * D + dv];
#pragma unroll
                for (int m = 0; m < PER; ++m) a[m] += sm.fk[rr * D + dk0 + DKS * m] * fvr;
            }
#pragma unroll
            for (int m = 0; m < PER; ++m) sm.S[(dk0 + DKS * m) * D + dv] += a[m];
            if (NORM && tid < D) {
                float a = 0.f;
                for (int rr = 0; rr < SUB; ++rr) a += sm.fk[rr * D + tid];
                sm.z[tid] += a;
            }
        }
    }
    if (it.last && it.row >= 0) {
        __syncthreads();
        if (state_out) {
            float* dst = state_out + ((size_t)it.row * H + h) * D * D;
            for (int e = tid; e < D * D; e += NT) dst[e] = sm.S[e];
        }
        if (NORM && z_out && tid < D) z_out[((size_t)it.row * H + h) * D + tid] = sm.z[tid];
    }
}

}  // namespace vk
}  // namespace la
