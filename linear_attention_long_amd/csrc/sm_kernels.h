// sm_kernels.h -- the softmax attention layer of the hybrid model (one layer
// in eight; the others are linear attention), head dim 128, bf16 inputs.
//
// Method: page "六十四：MiniMax-01" (LLM tutorial, lesson 64), sections 2-3:
// softmax(Q K^T / sqrt(d)) V, causal; page "MiniMax-Text-01 405B
// MoE模型架构与训练策略解析", section 2.2: rotary position embedding on half of
// each head's dimensions (base 10,000, raised to 5M and 10M in section 4.1);
// page "MiniMax-01系列大模型：超长上下文与多模态能力深度解析与部署指南",
// section 2.1.3: packed variable-length sequences.  Inside the first `rot`
// dimensions, dimension j pairs with j + rot/2 and turns by pos * base^(-2j/rot),
// positions counting from each sequence's start; query head h reads key/value
// head h / (H / Hkv).
//
// Three kernels per call:
//  * k_sm_plan (packed batches of more than one sequence): one workgroup
//    orders the (sequence, query tile) pairs by decreasing tile index, i.e.
//    by decreasing causal work, so the longest tiles start first;
//  * k_sm_rope: q and k are rotated once (angles reduced in fp64), scaled,
//    and rounded into the workspace (bf16, bf16 hi + lo, or fp16, by
//    precision mode; with fp16 operands v is scaled and rounded to fp16 as
//    well); every workgroup of the main kernel then reads ready operands;
//  * k_sm_attn: one workgroup = one (query tile, head); streaming softmax
//    over blocks of 128 keys (64 with split operands).
//
// gfx950 design of k_sm_attn:
//  * W = 8 waves x 32 queries (256-query tiles) in every precision mode, one
//    workgroup per CU, two waves per SIMD (fp16 operands use the single
//    layout with v_mfma_f32_16x16x32_f16 for both products).  Each staged
//    K/V block serves all W waves.
//    A wave's rotated Q stays in registers as MFMA operands for the whole
//    key loop;
//  * the score tile is produced transposed, S^T = K Q^T
//    (v_mfma_f32_16x16x32_bf16), so each lane holds 4 keys of one query: the
//    running max needs only two cross-lane steps;
//  * the running sum of the probabilities is taken over the same
//    bf16-rounded weights that multiply V, so numerator and denominator
//    agree: each lane adds its own keys' packed weights with
//    v_dot2_f32_bf16 against (1, 1) (products exact), and the four lane
//    groups of a query are added once, at the end;
//  * the k index of every MFMA is permuted so a lane's 8 slots are keys
//    {32s + 4g + i, 32s + 16 + 4g + i}: that is the order in which two
//    adjacent 16-key score tiles sit in a lane's accumulators, so the
//    probabilities feed O^T += V^T P^T straight from registers, converted to
//    bf16;
//  * K and V blocks are double-buffered in LDS (one barrier per block); the
//    next block's loads are in flight while the current one computes.  K is
//    read along rows (two 8-byte pieces per lane, merged into one
//    ds_read2_b64, row stride 132 elements: conflict-free), V with
//    transposing reads (ds_read_b64_tr_b16, row stride 144);
//  * scores are in log2 units (q carries log2(e)), so probabilities are one
//    v_exp_f32 each; the reference maximum m of a query is raised only when a
//    score exceeds it by more than 8 (probabilities then stay below 2^8), so
//    the rescale of the accumulators by exp2(m_old - m_new) is rare;
//  * K and V blocks arrive through buffer loads whose range ends at the
//    tile's last key (zeros past it, no per-lane bounds arithmetic);
//  * the matrix-core sections run at raised wave priority (s_setprio 1), so a
//    SIMD issues one wave's MFMA stream first and fills its gaps with the
//    other wave's vector work;
//  * 138 KiB of LDS per workgroup (102 KiB with split operands); the
//    blockIdx -> (tile, head) map puts key/value head hk on
//    XCD hk mod 8, so the workgroups sharing a head's K and V share that
//    XCD's L2.
#pragma once

#include "la_device.h"

namespace la {
namespace sm {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

constexpr int D = 128;    // head dim
// The attention kernel runs W waves of 32 queries each per workgroup: 64 W
// threads, a tile of 32 W queries.
template <int W>
struct Waves {
    static constexpr int NT = 64 * W;   // threads
    static constexpr int BQ = 32 * W;   // queries per tile
    static constexpr int RP = NT / 16;  // K/V rows staged per pass (16 threads per row)
};
#ifndef LA_SM_BLOCK
#define LA_SM_BLOCK 128
#endif
constexpr int kBlockPlain = LA_SM_BLOCK;  // keys per K/V block, single bf16 operands
constexpr int kBlockSplit = 64;           // keys per K/V block, split operands
constexpr int KSK = 132;  // LDS row stride of K (row reads)
constexpr int KSV = 144;  // LDS row stride of V (transposing reads)
constexpr int PADE = 8;   // elements after each LDS array (see the linear kernels)

// Double-buffered K and V blocks; with split operands also the bf16
// remainders of K.
template <bool SPLIT, int BN>
struct __attribute__((aligned(16))) Smem {
    __attribute__((aligned(16))) uint16_t k[2][BN * KSK + PADE];
    __attribute__((aligned(16))) uint16_t kl[SPLIT ? 2 : 1][SPLIT ? BN * KSK + PADE : 8];
    __attribute__((aligned(16))) uint16_t v[2][BN * KSV + PADE];
};

// ------------------------------------------------------------------ plan --

// Exclusive prefix sum over the 1024 threads of a workgroup; returns the sum
// of the values of lower threads and sets `total` to the sum over all.
__device__ __forceinline__ int block_excl_scan(int x, int& total, int* wsum /* [16] LDS */) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int inc = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(inc, o, 64);
        if (lane >= o) inc += y;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
        const int sw = wsum[w];
        before += w < wave ? sw : 0;
        all += sw;
    }
    __syncthreads();
    total = all;
    return before + inc - x;
}

// Orders the (sequence, query tile) pairs of a packed batch by decreasing
// tile index (ties in any order: each pair's result does not depend on when
// it runs).  Tile i of a sequence of length L exists for i < ceil(L / bq)
// (clamped to ntmax); the number of sequences with a tile i is
// cnt[i] = #{s : n_s > i}, the tiles with index i occupy table entries
// [off[i], off[i] + cnt[i]) with off[i] = sum of cnt[i'] over i' > i.
// One workgroup of 1024 threads.  Workspace arrays: hist [ntmax + 1],
// off and cursor [ntmax], tcu [nseq + 1].
__global__ __launch_bounds__(1024) void k_sm_plan(const int32_t* __restrict__ cu, int nseq,
                                                  int bq, int ntmax, int32_t* __restrict__ hist,
                                                  int32_t* __restrict__ off,
                                                  int32_t* __restrict__ cursor,
                                                  int32_t* __restrict__ tcu,
                                                  int2* __restrict__ table,
                                                  int32_t* __restrict__ ecount) {
    __shared__ int wsum[16];
    const int tid = threadIdx.x;
    for (int i = tid; i <= ntmax; i += 1024) {
        hist[i] = 0;
        if (i < ntmax) cursor[i] = 0;
    }
    __threadfence();
    __syncthreads();
    auto ntiles = [&](int s) {
        const int L = cu[s + 1] - cu[s];
        const int n = L > 0 ? (L + bq - 1) / bq : 0;
        return n < ntmax ? n : ntmax;
    };
    for (int s = tid; s < nseq; s += 1024) atomicAdd(&hist[ntiles(s)], 1);
    __threadfence();
    __syncthreads();
    // cnt and off in decreasing i: with r = ntmax - 1 - i, cnt = sum of
    // hist[n] over n >= ntmax - r (inclusive scan of hist read backwards),
    // off = exclusive scan of cnt in the same order.
    int carry_c = 0, carry_o = 0;
    for (int r0 = 0; r0 < ntmax; r0 += 1024) {
        const int r = r0 + tid;
        const int hv = r < ntmax ? __atomic_load_n(&hist[ntmax - r], __ATOMIC_RELAXED) : 0;
        int tot;
        const int c = carry_c + block_excl_scan(hv, tot, wsum) + hv;
        carry_c += tot;
        int tot2;
        const int o = carry_o + block_excl_scan(r < ntmax ? c : 0, tot2, wsum);
        carry_o += tot2;
        if (r < ntmax) off[ntmax - 1 - r] = o;
    }
    // per-sequence tile offsets (sequence order) for the flat enumeration
    int carry = 0;
    for (int s0 = 0; s0 < nseq; s0 += 1024) {
        const int s = s0 + tid;
        const int n = s < nseq ? ntiles(s) : 0;
        int tot;
        const int e = carry + block_excl_scan(n, tot, wsum);
        if (s < nseq) tcu[s] = e;
        carry += tot;
    }
    if (tid == 0) {
        tcu[nseq] = carry;
        *ecount = carry;
    }
    __threadfence();
    __syncthreads();
    const int E = carry;
    for (int f = tid; f < E; f += 1024) {
        int lo = 0, hi = nseq;  // largest s with tcu[s] <= f
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (tcu[mid] <= f) lo = mid; else hi = mid;
        }
        const int i = f - tcu[lo];
        const int slot = off[i] + atomicAdd(&cursor[i], 1);
        table[slot] = make_int2(lo, i);
    }
}

// ------------------------------------------------------------------ rope --

// Two floats as an fp16 pair (round to nearest even), first in the low half.
// A value past fp16's range (or an infinite input) is stored as NaN, not as
// an infinity: an infinite score can be -inf, which the softmax would take as
// a masked key, while a NaN reaches every output it touches.
__device__ __forceinline__ uint16_t f16_bits_or_nan(float a) {
    const uint16_t u = __builtin_bit_cast(uint16_t, (_Float16)a);
    return (u & 0x7fffu) == 0x7c00u ? (uint16_t)0x7e00u : u;
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    return (uint32_t)f16_bits_or_nan(a) | ((uint32_t)f16_bits_or_nan(b) << 16);
}

// Rotary embedding, scale and bf16 (or, for fp16 operands, fp16) rounding of q
// and k; q is multiplied by qscale and k by kscale before the rounding.  With
// vr (fp16 operands) v is also multiplied by vscale and rounded to fp16 into vr.
// 16 threads per token
// (thread u owns 8 dimensions), grid-stride over tokens; for each token the
// rotations are computed once and applied to its H query heads and Hkv key
// heads.  Thread u < rot/16 rotates dimensions [8u, 8u+8) with their partners
// [8u + rot/2, ...); threads with 8u >= rot copy (q: scale) their 8
// dimensions; the rest have no dimensions of their own.  The angle
// pos * theta_j is formed and reduced to [-pi, pi] in fp64, then sin and cos
// are taken in fp32.  rot is a multiple of 16 in [0, 128].
__global__ __launch_bounds__(256) void k_sm_rope(const uint16_t* __restrict__ q,
                                                 const uint16_t* __restrict__ k,
                                                 const int32_t* __restrict__ cu, int nseq, int T,
                                                 int H, int Hkv, int rot, double log2_base,
                                                 float qscale, float kscale,
                                                 uint16_t* __restrict__ qr,
                                                 uint16_t* __restrict__ kr,
                                                 uint16_t* __restrict__ qrl,
                                                 uint16_t* __restrict__ krl, int f16out,
                                                 const uint16_t* __restrict__ v,
                                                 uint16_t* __restrict__ vr, float vscale) {
    __shared__ double theta[64];
    if ((int)threadIdx.x < rot / 2)
        theta[threadIdx.x] = exp2(-(2.0 * (double)threadIdx.x / (double)rot) * log2_base);
    __syncthreads();
    const int u = threadIdx.x & 15;
    const int half = rot / 2;
    const bool pair = 8 * u < half;
    const bool plain = 8 * u >= rot;
    const double two_pi = 6.283185307179586476925;
    for (int64_t t = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4); t < T;
         t += (int64_t)gridDim.x * 16) {
        float cs[8], sn[8];
        if (pair) {
            int lo = 0, hi = nseq;  // sequence of token t: largest s with cu[s] <= t
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (cu[mid] <= t) lo = mid; else hi = mid;
            }
            const double pos = (double)(t - cu[lo]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const double a = pos * theta[8 * u + e];
                const double r = a - two_pi * rint(a * (1.0 / two_pi));
                sincosf((float)r, &sn[e], &cs[e]);
            }
        }
        for (int row = 0; row < H + Hkv; ++row) {
            const bool isq = row < H;
            const size_t base = isq ? ((size_t)t * H + row) * D : ((size_t)t * Hkv + (row - H)) * D;
            const uint16_t* src = (isq ? q : k) + base;
            uint16_t* dst = (isq ? qr : kr) + base;
            uint16_t* dlo = isq ? qrl : krl;  // bf16 remainders, or none
            if (dlo) dlo += base;
            const float sc = isq ? qscale : kscale;
            if (pair) {
                const uint4 wa = *(const uint4*)(src + 8 * u);
                const uint4 wb = *(const uint4*)(src + 8 * u + half);
                const uint32_t a32[4] = {wa.x, wa.y, wa.z, wa.w};
                const uint32_t b32[4] = {wb.x, wb.y, wb.z, wb.w};
                uint32_t oa[4], ob[4], la[4], lb[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const float a0 = bf16_lo_to_f32(a32[p]), a1 = bf16_hi_to_f32(a32[p]);
                    const float b0 = bf16_lo_to_f32(b32[p]), b1 = bf16_hi_to_f32(b32[p]);
                    const float c0 = cs[2 * p], s0 = sn[2 * p], c1 = cs[2 * p + 1], s1 = sn[2 * p + 1];
                    const float ra0 = (a0 * c0 - b0 * s0) * sc, ra1 = (a1 * c1 - b1 * s1) * sc;
                    const float rb0 = (b0 * c0 + a0 * s0) * sc, rb1 = (b1 * c1 + a1 * s1) * sc;
                    if (f16out) {
                        oa[p] = pack_f16x2(ra0, ra1);
                        ob[p] = pack_f16x2(rb0, rb1);
                    } else {
                        split2_keep(ra0, ra1, oa[p], la[p]);
                        split2_keep(rb0, rb1, ob[p], lb[p]);
                    }
                }
                *(uint4*)(dst + 8 * u) = make_uint4(oa[0], oa[1], oa[2], oa[3]);
                *(uint4*)(dst + 8 * u + half) = make_uint4(ob[0], ob[1], ob[2], ob[3]);
                if (dlo) {
                    *(uint4*)(dlo + 8 * u) = make_uint4(la[0], la[1], la[2], la[3]);
                    *(uint4*)(dlo + 8 * u + half) = make_uint4(lb[0], lb[1], lb[2], lb[3]);
                }
            } else if (plain) {
                const uint4 w = *(const uint4*)(src + 8 * u);
                const uint32_t w32[4] = {w.x, w.y, w.z, w.w};
                uint32_t o[4], lo[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    if (f16out)
                        o[p] = pack_f16x2(bf16_lo_to_f32(w32[p]) * sc, bf16_hi_to_f32(w32[p]) * sc);
                    else
                        split2_keep(bf16_lo_to_f32(w32[p]) * sc, bf16_hi_to_f32(w32[p]) * sc, o[p], lo[p]);
                }
                *(uint4*)(dst + 8 * u) = make_uint4(o[0], o[1], o[2], o[3]);
                if (dlo) *(uint4*)(dlo + 8 * u) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
            }
        }
        if (vr) {  // every thread converts its 8 dimensions of each value head
            for (int hv = 0; hv < Hkv; ++hv) {
                const size_t base = ((size_t)t * Hkv + hv) * D + 8 * u;
                const uint4 w = *(const uint4*)(v + base);
                const uint32_t w32[4] = {w.x, w.y, w.z, w.w};
                uint32_t o[4];
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    o[p] = pack_f16x2(bf16_lo_to_f32(w32[p]) * vscale, bf16_hi_to_f32(w32[p]) * vscale);
                *(uint4*)(vr + base) = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
    }
}

// ------------------------------------------------------------- attention --

template <typename OutT>
__device__ __forceinline__ void store_out4(OutT* p, f32x4_t v, float s);
template <>
__device__ __forceinline__ void store_out4<float>(float* p, f32x4_t v, float s) {
    *(f32x4_t*)p = v * s;
}
template <>
__device__ __forceinline__ void store_out4<uint16_t>(uint16_t* p, f32x4_t v, float s) {
    *(uint2*)p = make_uint2(cvt_pk_bf16(v[0] * s, v[1] * s), cvt_pk_bf16(v[2] * s, v[3] * s));
}

// Sum of eight bf16 values (four packed pairs) into an fp32 accumulator: one
// v_dot2_f32_bf16 against (1, 1) per pair, products exact.
__device__ __forceinline__ float sum8_bf16(uint4 u, float acc) {
    const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, u.x), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, u.y), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, u.z), one, acc, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, u.w), one, acc, false);
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed fp16 (round to nearest even), one v_cvt_pk_f16_f32.
__device__ __forceinline__ uint32_t cvt_pk_f16(float a, float b) {
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

// The fp16 form of sum8_bf16: one v_dot2_f32_f16 against (1, 1) per pair.
__device__ __forceinline__ float sum8_f16(uint4 u, float acc) {
    const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, u.x), one, acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, u.y), one, acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, u.z), one, acc, false);
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, u.w), one, acc, false);
}

// Operand of 32 head dimensions of one LDS row for the permuted k order:
// columns {k0 + 4g + i, k0 + 16 + 4g + i}; the literal 16 lets the compiler
// merge the two 8-byte reads into one ds_read2_b64.
__device__ __forceinline__ bf16x8_t k_operand(const uint16_t* tile, int row, int k0, int g) {
    const uint16_t* p = tile + row * KSK + k0 + 4 * g;
    return as_bf16x8(lds_read8(p), lds_read8(p + 16));
}

// Operand over 32 keys (rows of the row-major V tile) for the permuted k
// order: lane (g, c) gets column c0 + c, rows {r0 + 4g + i, r0 + 16 + 4g + i}.
__device__ __forceinline__ bf16x8_t v_operand(const uint16_t* tile, int r0, int c0, int g, int c) {
    return as_bf16x8(lds_read_tr4(tile, KSV, r0 + 4 * g, c0, c),
                     lds_read_tr4(tile, KSV, r0 + 16 + 4 * g, c0, c));
}

// One (32 W-query tile, query head) of causal softmax attention.
//   qr [T, H, D] bf16: rotated q times scale * log2(e); kr [T, Hkv, D] bf16:
//   rotated k; v [T, Hkv, D] bf16; out [T, H, D]; lse [T, H] (natural log)
//   or null.  table/ecount: the plan (null for a single sequence, whose
//   tiles then run last tile first).
// SPLIT: qrl, krl hold the bf16 remainders (x - bf16(x)) of the rotated q and
// k, and q is NOT pre-scaled: the scores are multiplied by qs (scale * log2 e)
// in fp32.  Dimensions past the rotated ones are then exact in bf16 on both
// sides (the inputs are bf16), so the 32-dimension steps kk >= NRK (NRK =
// ceil(rot / 32)) take one product and the rotated steps three
// (hi.hi + lo.hi + hi.lo); the probabilities are split into bf16 hi + lo for
// two products with V (V is exact).  Both contractions keep ~16 significant
// bits.  Without SPLIT, q carries the scale and NRK is unused.
// F16 (without SPLIT): fp16 operands -- qr and kr hold the rotated q and k
// times 2^-6 each, v holds the values times 2^-6, all fp16; one fp16 product
// per score (qs then carries 2^12 and is applied in fp32 as with SPLIT) and
// one per P V step, the probabilities rounded to fp16; ovs (2^6) scales the
// output back.  ovs is 1 in the other modes.
template <typename OutT, bool SPLIT, int W, int NRK = 4, bool F16 = false>
__global__ __launch_bounds__(64 * W, (SPLIT || W == 8) ? 1 : 2) void k_sm_attn(const uint16_t* __restrict__ qr,
                                                   const uint16_t* __restrict__ kr,
                                                   const uint16_t* __restrict__ qrl,
                                                   const uint16_t* __restrict__ krl,
                                                   const uint16_t* __restrict__ v,
                                                   const int32_t* __restrict__ cu,
                                                   const int2* __restrict__ table,
                                                   const int32_t* __restrict__ ecount, int H,
                                                   int Hkv, OutT* __restrict__ out,
                                                   float* __restrict__ lse, float qs, float ovs) {
    static_assert(NRK >= 0 && NRK <= 4, "rotated 32-dimension steps");
    static_assert(!F16 || !SPLIT, "fp16 operands: single products");
    constexpr bool KLO = SPLIT && NRK > 0;  // bf16 remainders of k staged and used
    constexpr int BN = SPLIT ? kBlockSplit : kBlockPlain;  // keys per K/V block
    constexpr int NKT = BN / 16;  // 16-key score tiles per block
    constexpr int NKS = BN / 32;  // 32-key steps of the P V product
    __shared__ Smem<KLO, BN> sm;
    constexpr int BQ = Waves<W>::BQ, RP = Waves<W>::RP, NJ = BN / RP;
    const int G = H / Hkv;
    const int b = blockIdx.x;
    const int hk = b % Hkv;
    const int rest = b / Hkv;
    const int h = hk * G + rest % G;
    const int e = rest / G;
    int s, ti;
    if (table == nullptr) {
        const int L0 = cu[1] - cu[0];
        const int nt = (L0 + BQ - 1) / BQ;
        if (e >= nt) return;
        s = 0;
        ti = nt - 1 - e;
    } else {
        if (e >= *ecount) return;
        const int2 it = table[e];
        s = it.x;
        ti = it.y;
    }
    const int start = cu[s];
    const int L = cu[s + 1] - start;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int q0 = ti * BQ;
    if (q0 >= L) return;  // (only if a length exceeds the plan's bound)
    const int kv_end = min(L, q0 + BQ);
    const int nblk = (kv_end + BN - 1) / BN;
    const int wq0 = q0 + 32 * wave;          // this wave's first query
    const bool has_q = wq0 < L;
    const int wq_last = min(wq0 + 31, L - 1);

    // Q^T operands: lane (g, c) holds query wq0 + 16 qt + c, dimensions
    // {32 kk + 4g + i, 32 kk + 16 + 4g + i}.
    constexpr int NQL = (SPLIT && NRK > 0) ? NRK : 1;  // steps with a q remainder
    bf16x8_t Qf[2][4], Ql[2][NQL];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const int row = wq0 + 16 * qt + c;
        const size_t off = ((size_t)(start + row) * H + h) * D + 4 * g;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            i16x4_t lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
            if (row < L) {
                lo = *(const i16x4_t*)(qr + off + 32 * kk);
                hi = *(const i16x4_t*)(qr + off + 32 * kk + 16);
            }
            Qf[qt][kk] = as_bf16x8(lo, hi);
            if constexpr (SPLIT) {
                if (kk < NRK) {
                    i16x4_t lo2 = {0, 0, 0, 0}, hi2 = {0, 0, 0, 0};
                    if (row < L) {
                        lo2 = *(const i16x4_t*)(qrl + off + 32 * kk);
                        hi2 = *(const i16x4_t*)(qrl + off + 32 * kk + 16);
                    }
                    Ql[qt][kk < NQL ? kk : 0] = as_bf16x8(lo2, hi2);
                }
            }
        }
    }

    // O^T accumulators; lsum[qt]: this lane's part (its keys 4g + i of every
    // 16-key tile) of the query's sum of the same rounded weights that
    // multiply V; the four lane groups are added at the end.
    f32x4_t O[8][2];
    float lsum[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        lsum[qt] = 0.f;
#pragma unroll
        for (int ft = 0; ft < 8; ++ft) O[ft][qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // Reference maximum per query (log2 units).  Probabilities are exp2(s - m)
    // with m raised only when a score exceeds it by more than kLazy, so the
    // accumulators are rescaled rarely; they stay below 2^kLazy.
    constexpr float kLazy = 8.0f;
    float m[2] = {-1e30f, -1e30f};

    // staging: thread tid moves rows (tid >> 4) + 16 j, dimensions
    // (tid & 15) * 8 .. + 7 of the 64-key block through buffer loads whose
    // range ends at kv_end: keys past it (after every query of the tile,
    // so masked) read as zeros.
    const uint32_t rs = (uint32_t)(Hkv * D);
    const uint16_t* kseq = kr + ((size_t)start * Hkv + hk) * D;
    const uint16_t* vseq = v + ((size_t)start * Hkv + hk) * D;
    const uint16_t* klseq = KLO ? krl + ((size_t)start * Hkv + hk) * D : nullptr;
    const uint32_t voff = ((uint32_t)(tid >> 4) * rs + (uint32_t)(tid & 15) * 8) * 2u;
    // the remainders of k are zero past the rotated dimensions: only the
    // threads whose 8 dimensions lie in the first 32 NRK move them
    const bool klo_thread = KLO && (tid & 15) < 4 * NRK;
    uint4 rk[NJ], rv[NJ], rkl[KLO ? NJ : 1];
    auto load_kv = [&](int blk) {
        const int nvalid = kv_end - blk * BN;
        const int32_t bytes = (int32_t)((uint32_t)(min(nvalid, BN) - 1) * rs * 2u + 2u * D);
        const size_t base = (size_t)blk * BN * rs;
        const __amdgpu_buffer_rsrc_t rsk =
            __builtin_amdgcn_make_buffer_rsrc((void*)(kseq + base), (short)0, bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rsv =
            __builtin_amdgcn_make_buffer_rsrc((void*)(vseq + base), (short)0, bytes, 0x00020000);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            rk[j] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(rsk, voff + (uint32_t)(RP * j) * rs * 2u, 0, 0));
            rv[j] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(rsv, voff + (uint32_t)(RP * j) * rs * 2u, 0, 0));
        }
        if constexpr (KLO) {
            if (klo_thread) {
                const __amdgpu_buffer_rsrc_t rskl =
                    __builtin_amdgcn_make_buffer_rsrc((void*)(klseq + base), (short)0, bytes, 0x00020000);
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    rkl[j] = __builtin_bit_cast(
                        uint4, __builtin_amdgcn_raw_buffer_load_b128(rskl, voff + (uint32_t)(RP * j) * rs * 2u, 0, 0));
            }
        }
    };
    auto store_kv = [&](int buf) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int r = (tid >> 4) + RP * j;
            uint2* pk = (uint2*)(sm.k[buf] + r * KSK + (tid & 15) * 8);
            pk[0] = make_uint2(rk[j].x, rk[j].y);
            pk[1] = make_uint2(rk[j].z, rk[j].w);
            *(uint4*)(sm.v[buf] + r * KSV + (tid & 15) * 8) = rv[j];
            if constexpr (KLO) {
                if (klo_thread) {
                    uint2* pl = (uint2*)(sm.kl[buf] + r * KSK + (tid & 15) * 8);
                    pl[0] = make_uint2(rkl[j].x, rkl[j].y);
                    pl[1] = make_uint2(rkl[j].z, rkl[j].w);
                }
            }
        }
    };

    load_kv(0);
    store_kv(0);
    __syncthreads();
    for (int blk = 0; blk < nblk; ++blk) {
        const int buf = blk & 1;
        if (blk + 1 < nblk) load_kv(blk + 1);
        const int kb0 = blk * BN;
        if (has_q && kb0 <= wq_last) {
            // S^T tiles: Sc[kt][qt], lane (g, c) = query wq0 + 16 qt + c,
            // keys kb0 + 16 kt + 4g + i.
            f32x4_t Sc[NKT][2];
            const uint16_t* kt_ = sm.k[buf];
            __builtin_amdgcn_s_setprio(1);  // matrix-core section (see below)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) {
                    const bf16x8_t A = k_operand(kt_, 16 * kt + c, 32 * kk, g);
#pragma unroll
                    for (int qt = 0; qt < 2; ++qt) {
                        const f32x4_t c0 = kk == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : Sc[kt][qt];
                        if constexpr (F16)  // q and k held as fp16 (the same 16-bit lanes)
                            Sc[kt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                __builtin_bit_cast(f16x8_t, A), __builtin_bit_cast(f16x8_t, Qf[qt][kk]), c0, 0, 0, 0);
                        else
                            Sc[kt][qt] = mfma16x16x32(A, Qf[qt][kk], c0);
                    }
                    if constexpr (KLO) {  // rotated steps: + k_lo . q_hi + k_hi . q_lo
                        if (kk < NRK) {
                            const bf16x8_t Al = k_operand(sm.kl[buf], 16 * kt + c, 32 * kk, g);
#pragma unroll
                            for (int qt = 0; qt < 2; ++qt) {
                                Sc[kt][qt] = mfma16x16x32(Al, Qf[qt][kk], Sc[kt][qt]);
                                Sc[kt][qt] = mfma16x16x32(A, Ql[qt][kk < NQL ? kk : 0], Sc[kt][qt]);
                            }
                        }
                    }
                }
            __builtin_amdgcn_s_setprio(0);
            // scores in log2 units are Sc * sc: with split or fp16 operands
            // the unscaled products (sc = qs > 0, applied below inside the
            // exponent's argument and to the block maximum), else q carries it
            const float sc = (SPLIT || F16) ? qs : 1.0f;
            if (kb0 + BN - 1 > wq0) {  // causal mask on the diagonal blocks
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) {
                    const int qi = wq0 + 16 * qt + c;
#pragma unroll
                    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (kb0 + 16 * kt + 4 * g + i > qi) Sc[kt][qt][i] = -INFINITY;
                }
            }
            // streaming softmax (log2 units)
            float mx[2];
            bool raise = false;
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                float x = Sc[0][qt][0];
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) x = fmaxf(x, Sc[kt][qt][i]);
                x = fmaxf(x, __shfl_xor(x, 16, 64));
                mx[qt] = fmaxf(x, __shfl_xor(x, 32, 64)) * sc;
                raise |= mx[qt] > m[qt] + kLazy;
            }
            if (__builtin_amdgcn_ballot_w64(raise)) {
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) {
                    const float mn = mx[qt] > m[qt] + kLazy ? mx[qt] : m[qt];
                    const float alpha = __builtin_amdgcn_exp2f(m[qt] - mn);
                    m[qt] = mn;
                    lsum[qt] *= alpha;
#pragma unroll
                    for (int ft = 0; ft < 8; ++ft) O[ft][qt] *= alpha;
                }
            }
#pragma unroll
            for (int qt = 0; qt < 2; ++qt)
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        Sc[kt][qt][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(Sc[kt][qt][i], sc, -m[qt]));
            // P^T operands: keys {32 ks + 4g + i} from tile 2ks, {32 ks + 16 + 4g + i}
            // from tile 2ks + 1.
            bf16x8_t Pf[NKS][2], Pl[SPLIT ? NKS : 1][2];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) {
                    const f32x4_t a = Sc[2 * ks][qt], bq = Sc[2 * ks + 1][qt];
                    if constexpr (SPLIT) {
                        uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
                        split2(a[0], a[1], h0, l0);
                        split2(a[2], a[3], h1, l1);
                        split2(bq[0], bq[1], h2, l2);
                        split2(bq[2], bq[3], h3, l3);
                        Pf[ks][qt] = as_bf16x8(make_uint4(h0, h1, h2, h3));
                        Pl[ks][qt] = as_bf16x8(make_uint4(l0, l1, l2, l3));
                        lsum[qt] = sum8_bf16(make_uint4(l0, l1, l2, l3),
                                             sum8_bf16(make_uint4(h0, h1, h2, h3), lsum[qt]));
                    } else if constexpr (F16) {
                        const uint4 p4 = make_uint4(cvt_pk_f16(a[0], a[1]), cvt_pk_f16(a[2], a[3]),
                                                    cvt_pk_f16(bq[0], bq[1]), cvt_pk_f16(bq[2], bq[3]));
                        Pf[ks][qt] = as_bf16x8(p4);  // fp16 bits in the 16-bit lanes
                        lsum[qt] = sum8_f16(p4, lsum[qt]);
                    } else {
                        const uint4 p4 = make_uint4(cvt_pk_bf16(a[0], a[1]), cvt_pk_bf16(a[2], a[3]),
                                                    cvt_pk_bf16(bq[0], bq[1]), cvt_pk_bf16(bq[2], bq[3]));
                        Pf[ks][qt] = as_bf16x8(p4);
                        lsum[qt] = sum8_bf16(p4, lsum[qt]);
                    }
                }
            const uint16_t* vt_ = sm.v[buf];
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
                for (int ft = 0; ft < 8; ++ft) {
                    const bf16x8_t A = v_operand(vt_, 32 * ks, 16 * ft, g, c);
#pragma unroll
                    for (int qt = 0; qt < 2; ++qt) {
                        if constexpr (F16)
                            O[ft][qt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                __builtin_bit_cast(f16x8_t, A), __builtin_bit_cast(f16x8_t, Pf[ks][qt]),
                                O[ft][qt], 0, 0, 0);
                        else
                            O[ft][qt] = mfma16x16x32(A, Pf[ks][qt], O[ft][qt]);
                        if constexpr (SPLIT) O[ft][qt] = mfma16x16x32(A, Pl[ks][qt], O[ft][qt]);
                    }
                }
            }
            __builtin_amdgcn_s_setprio(0);
        }
        if (blk + 1 < nblk) store_kv(buf ^ 1);
        __syncthreads();
    }

    // normalise and store: lane (g, c) holds features 16 ft + 4g + i of query
    // wq0 + 16 qt + c.
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        float lt = lsum[qt] + __shfl_xor(lsum[qt], 16, 64);
        lt += __shfl_xor(lt, 32, 64);
        const int row = wq0 + 16 * qt + c;
        if (row < L) {
            const float inv = ovs / lt;
            OutT* op = out + ((size_t)(start + row) * H + h) * D + 4 * g;
#pragma unroll
            for (int ft = 0; ft < 8; ++ft) store_out4<OutT>(op + 16 * ft, O[ft][qt], inv);
            if (lse != nullptr && g == 0)
                lse[(size_t)(start + row) * H + h] = (m[qt] + __log2f(lt)) * 0.69314718055994530942f;
        }
    }
}

}  // namespace sm
}  // namespace la
