// proj_kernels.h -- the input projection of a lightning-attention layer as one
// bf16 matrix-core GEMM with the feature map in its epilogue (gfx950).
//
// Page "MiniMax-Text-01 405B MoE模型架构与训练策略解析", section 2.1: Q, K, V =
// SiLU of the layer input's projections, and the output gate sigmoid(.) of a
// projection of its own.  For one GPU's heads (F = H * d features per token):
//     P = hidden @ W^T,   W = [W_q; W_k; W_v; W_g]  ([nblk * F, K], rows = output features)
//     q, k, v = SiLU(P[:, 0:F]), SiLU(P[:, F:2F]), SiLU(P[:, 2F:3F]);  x_gate = P[:, 3F:4F]
// written as four [tokens, F] tensors, i.e. q, k, v in the [tokens, H, d]
// layout the attention path reads.
//
// gfx950 design:
//  * one workgroup = 8 waves = a 256 (features) x 256 (tokens) output tile;
//    wave w computes 128 x 64 of it as 8 x 4 tiles of v_mfma_f32_16x16x32_bf16
//    (32 accumulators of 4 fp32 per lane), two waves per SIMD, so one wave's
//    LDS reads overlap the other's matrix-core work (4 waves of 128 x 128, one
//    per SIMD, fit with their 256 accumulators in AGPRs but measured 43%
//    against 48% of the bf16 peak: a lone wave cannot hide its own LDS
//    latency);
//  * the weight is the MFMA A operand (rows = output features) and the hidden
//    states the B operand (columns = tokens), so a lane's accumulator holds 4
//    consecutive output features of one token: one 8-byte (bf16) or 16-byte
//    (fp32) store;
//  * both operand tiles stream through LDS in 64-wide reduction slices,
//    double-buffered (128 KB), one barrier per slice, loaded straight from
//    global memory into LDS (buffer_load_dwordx4 ... lds: no staging
//    registers); such a
//    load writes 16 bytes per lane at consecutive LDS addresses, so rows are
//    unpadded (128 bytes) and each lane instead fetches the global 16-byte
//    chunk that belongs in its slot: chunk s of row r sits in slot s ^ (r & 7).
//    The 16-byte fragment reads of eight consecutive rows then hit eight
//    distinct slots, i.e. distinct banks;
//  * the next slice's loads (zero past the last token) are in flight while the
//    current slice's 64 MFMAs per wave run.  Measured alternatives that did
//    not pay: a ring of 4 or 5 LDS stages of 32-wide slices (loads three or
//    four steps ahead: no gain, so load latency is not the limit) and
//    v_mfma_f32_32x32x16_bf16 tiles (same LDS traffic, a few % slower);
//  * blockIdx -> tile is XCD-aware: workgroup i runs on XCD i % 8, and each XCD
//    takes a contiguous range of tiles, ordered in groups of 4 token tiles per
//    feature tile so that the concurrently running workgroups of an XCD (4
//    token tiles x 8 feature tiles) share their weight and hidden-state
//    slices in that XCD's L2 (measured against groups of 2 to 32: 3 to 6
//    are within 1% of each other, 8 is 5-15% slower, 16 and 32 slower still).
#pragma once

#include "la_device.h"

namespace la {
namespace pj {

constexpr int BM = 256;      // tokens per workgroup tile
constexpr int BN = 256;      // output features per workgroup tile
constexpr int BK = 64;       // reduction slice per LDS stage (one 128-byte row)
constexpr int NT = 512;      // threads (8 waves)
constexpr int GM = 4;        // token tiles per group in the tile order

struct __attribute__((aligned(1024))) Smem {
    __attribute__((aligned(1024))) uint16_t w[2][BN * BK];
    __attribute__((aligned(1024))) uint16_t x[2][BM * BK];
};

typedef __attribute__((address_space(3))) void lds_void_t;

struct Args {
    const uint16_t* x;  // hidden states [M, K] bf16
    const uint16_t* w;  // weight [nblk * F, K] bf16, row n = output feature n
    void* out[4];       // q, k, v, x_gate: [M, F] each (out[3] unused when nblk = 3)
    int M, K, F;
    int nsilu;          // output blocks [0, nsilu) get the feature map
    int tiles_m, tiles_n, per_xcd;
};

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    // word 3: gfx9-family raw buffer (32-bit data format, no swizzle)
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int32_t)bytes, 0x00020000);
}

template <typename OutT>
__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t r, uint32_t elem, f32x4_t v);
template <>
__device__ __forceinline__ void store4<float>(__amdgpu_buffer_rsrc_t r, uint32_t elem, f32x4_t v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, elem * 4u, 0, 0);
}
template <>
__device__ __forceinline__ void store4<uint16_t>(__amdgpu_buffer_rsrc_t r, uint32_t elem, f32x4_t v) {
    const u32x2_t u = {cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3])};
    __builtin_amdgcn_raw_buffer_store_b64(u, r, elem * 2u, 0, 0);
}

template <typename OutT>
__global__ __launch_bounds__(NT, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_proj(Args a) {
    __shared__ Smem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c = lane & 15;
    const int wn = wave >> 2, wm = wave & 3;  // wave's 128 features and 64 tokens

    // tile of this workgroup (XCD-aware order, see the header)
    const int t = (blockIdx.x & 7) * a.per_xcd + (int)(blockIdx.x >> 3);
    if (t >= a.tiles_m * a.tiles_n) return;
    const int grp = t / (GM * a.tiles_n);
    const int r = t - grp * GM * a.tiles_n;
    const int rows_in_grp = min(GM, a.tiles_m - grp * GM);
    const int mt = grp * GM + r % rows_in_grp, nt = r / rows_in_grp;
    const int m0 = mt * BM, n0 = nt * BN;
    const int mvalid = min(BM, a.M - m0);

    const uint32_t rowb = (uint32_t)a.K * 2u;  // bytes per row of x and w
    const __amdgpu_buffer_rsrc_t rx = rsrc(a.x + (size_t)m0 * a.K, (uint32_t)mvalid * rowb);
    const __amdgpu_buffer_rsrc_t rw = rsrc(a.w + (size_t)n0 * a.K, (uint32_t)BN * rowb);

    // staging: wave w fills row groups w + 8j (8 rows, 1 KB each), j < 4, of
    // both tiles; lane l writes slot l % 8 of row 8 (w + 8j) + l / 8, which
    // holds the row's global chunk (l % 8) ^ (l / 8)
    const uint32_t lrow = (uint32_t)lane >> 3;
    const uint32_t lchunk = ((uint32_t)lane & 7) ^ lrow;
    auto gload = [&](int kt, int buf) {
        const uint32_t kb = (uint32_t)(kt * BK) * 2u + lchunk * 16u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int grp8 = wave + 8 * j;
            const uint32_t off = (uint32_t)(8 * grp8 + lrow) * rowb + kb;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)&sm.x[buf][grp8 * 8 * BK], 16, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void_t*)&sm.w[buf][grp8 * 8 * BK], 16, off, 0, 0, 0);
        }
    };

    f32x4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[i][jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // fragment rows: row 16 i + c of the wave's feature rows and token rows;
    // chunk kc of such a row sits in slot kc ^ (c & 7)
    const int wrow = 128 * wn + c, xrow = 64 * wm + c;
    auto fragments = [&](int buf, int ks, bf16x8_t (&A)[8], bf16x8_t (&B)[4]) {
        const int slot = ((4 * ks + g) ^ (c & 7)) * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) A[i] = *(const bf16x8_t*)(sm.w[buf] + (wrow + 16 * i) * BK + slot);
#pragma unroll
        for (int i = 0; i < 4; ++i) B[i] = *(const bf16x8_t*)(sm.x[buf] + (xrow + 16 * i) * BK + slot);
    };
    auto products = [&](const bf16x8_t (&A)[8], const bf16x8_t (&B)[4]) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) acc[i][jj] = mfma16x16x32(A[i], B[jj], acc[i][jj]);
    };

    // Two k-steps of 32 per slice.  Iteration kt: the fragments of its second
    // step are read while the first step's products run; then the barrier
    // (every wave's reads of buffer kt & 1 done, every wave's loads of slice
    // kt + 1 landed), the loads of slice kt + 2 into the freed buffer, and the
    // first step's fragments of slice kt + 1 read while the second step's
    // products run, so a slice's loads have a whole iteration to land.  The
    // body has no branches: the last iterations load slices past K (zeros past
    // the last row, into a buffer nobody reads again) and read fragments they
    // never use.
    const int nk = a.K / BK;
    bf16x8_t A0[8], B0[4], A1[8], B1[4];
    gload(0, 0);
    gload(1, 1);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    fragments(0, 0, A0, B0);
    // Issue order inside each half (sched_group_barrier; masks: 0x008 MFMA,
    // 0x010 memory loads, 0x100 LDS reads): the 12 fragment reads go one per
    // product at the head of the half, so they land well before the next
    // half needs them; after the barrier the 8 slice loads go first, one per
    // two products.  Issued in bursts instead (reads all ahead of the
    // products, the loads back to back) the same loop runs ~8% slower
    // (measured: 52% against 48% of the bf16 peak at 32768 x 6144 x 4096).
    // sched_barrier(0) fences keep each half's reads ahead of products that
    // do not depend on them; left alone, the scheduler sinks the reads next
    // to their consumers, past the loop's back edge.
    for (int kt = 0; kt < nk; ++kt) {
        const int b = kt & 1;
        fragments(b, 1, A1, B1);
        products(A0, B0);
#pragma unroll
        for (int i = 0; i < 12; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 20, 0);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        gload(kt + 2, b);
        fragments(b ^ 1, 0, A0, B0);
        products(A1, B1);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x010, 1, 1);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
        }
#pragma unroll
        for (int i = 0; i < 12; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
        __builtin_amdgcn_sched_barrier(0);
    }

    // epilogue: acc[i][jj][e] = P[token m0 + 64 wm + 16 jj + c][feature n0 + 128 wn + 16 i + 4 g + e]
    const int blk = n0 / a.F;  // a tile lies in one output block (F % BN == 0)
    const int fcol = n0 - blk * a.F + 128 * wn + 4 * g;
    const bool feat = blk < a.nsilu;
    const __amdgpu_buffer_rsrc_t ro =
        rsrc((const OutT*)a.out[blk] + (size_t)m0 * a.F, (uint32_t)mvalid * a.F * sizeof(OutT));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            f32x4_t v = acc[i][jj];
            if (feat) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = silu(v[e]);
            }
            const uint32_t row = 64 * wm + 16 * jj + c;
            store4<OutT>(ro, row * (uint32_t)a.F + fcol + 16 * i, v);
        }
    }
}

}  // namespace pj
}  // namespace la
