// la_kernels_mfma.h -- bf16 matrix-core (MFMA) kernels for head dim 128.
//
// Method (page "MiniMax-Text-01 405B MoE模型架构与训练策略解析" section 2.1 and
// page "六十四：MiniMax-01" section 3): per head, phi = SiLU on q, k, v;
// y_t = phi(q_t)^T S_t with S_t = S_{t-1} + phi(k_t) phi(v_t)^T, the sum
// including token t.  Evaluated in blocks of TB = 32 or 64 tokens: inside a block the
// masked quadratic form (phi(Q) phi(K)^T (.) M) phi(V), M = lower triangle
// with the diagonal; across blocks phi(Q) S_prev with the fp32 state carried
// in registers; after the block S += phi(K)^T phi(V).
//
// gfx950 design:
//  * one workgroup = 4 waves = one (chunk, head); with TB = 32 the LDS of a
//    workgroup is ~64 KB and two workgroups share a CU, so one's SiLU/split
//    VALU work overlaps the other's matrix-core work; wave w owns value columns
//    [32w, 32w+32) of the state (128 x 32 fp32 = 64 accumulator registers per
//    lane) and of the output, so the state never leaves registers;
//  * q, k, v of a block are staged once into LDS as bf16 hi/lo pairs
//    of phi(x) (hi = RNE(phi), lo = RNE(phi - hi)), row-major;
//  * every product takes three bf16 MFMAs (hi*hi + hi*lo + lo*hi), which
//    carries ~16 significant bits of each operand: with single bf16 operands
//    the intra-block term alone (all of y for short sequences) is off by
//    ~1.5e-2 of rms;
//  * LDS traffic is arranged to be free of bank conflicts (measured with the
//    SQ_LDS_BANK_CONFLICT counter on gfx950): contractions over tokens read
//    transposed fragments with ds_read_b64_tr_b16 from row-major K, V and P^T
//    tiles at a row stride of 144 (K, V) or TB + 16 (P^T) elements, each 16-lane
//    group covering four consecutive rows; contractions over the head dim
//    read two 8-byte pieces per lane (never 16-byte row reads, which conflict)
//    from Q and K rows.  The k index of every MFMA is permuted so that a
//    lane's 8 slots are {32s + 4g + i, 32s + 16 + 4g + i}, i < 4, which is
//    also the order in which a lane holds the fp32 state (C layout), so the
//    state feeds the inter-block product straight from registers;
//  * outputs are produced transposed (Y^T = V^T P^T + S^T Q^T) so each lane
//    holds 4 consecutive output features and stores 16 bytes;
//  * the next block's raw q, k, v are loaded into registers while the
//    current block computes.
#pragma once

#include "la_device.h"
#include "la_items.h"

namespace la {
namespace mf {

constexpr int D = 128;   // head dim
constexpr int NT = 256;  // threads per workgroup
constexpr int QS = 136;  // LDS row stride of the Q tile (bf16 elements)
constexpr int KS = 144;  // LDS row stride of the K and V tiles
// 16 bytes after each LDS array: neighbouring hi/lo arrays then are not a
// multiple of 512 bytes apart, so the compiler cannot fuse a read of one with
// a read of the other into a ds_read2st64 that lands both halves in the same
// banks.
constexpr int APAD = 8;

template <int TB>
struct Tile {
    static_assert(TB == 32 || TB == 64, "block of 32 or 64 tokens");
    static constexpr int PS = TB + 16;   // LDS row stride of P^T ([key][query])
    static constexpr int NJ = TB / 16;   // staged rows per thread
    static constexpr int NQT = TB / 16;  // 16-row query tiles
    static constexpr int NKS = TB / 32;  // 32-key steps
    static constexpr int WG_PER_CU = TB == 32 ? 2 : 1;
};

template <int TB>
struct __attribute__((aligned(16))) SmemMain {
    __attribute__((aligned(16))) uint16_t qh[TB * QS + APAD];
    __attribute__((aligned(16))) uint16_t ql[TB * QS + APAD];
    __attribute__((aligned(16))) uint16_t kh[TB * KS + APAD];
    __attribute__((aligned(16))) uint16_t kl[TB * KS + APAD];
    __attribute__((aligned(16))) uint16_t vh[TB * KS + APAD];
    __attribute__((aligned(16))) uint16_t vl[TB * KS + APAD];
    __attribute__((aligned(16))) uint16_t ph[TB * Tile<TB>::PS + APAD];  // P^T[key][query], hi
    __attribute__((aligned(16))) uint16_t pl[TB * Tile<TB>::PS + APAD];  // P^T[key][query], lo
    float denp[Tile<TB>::NQT * TB];  // normalised mode: row sums of P per 16-key tile
    float zq[TB];                    // normalised mode: phi(q) . z_prev per row
    float zpart[4 * D];              // normalised mode: column sums of phi(k) per wave
    float z[D];                      // normalised mode: running normaliser
    // fused gate (32-token blocks only; a stub of one element otherwise)
    static constexpr int FB = TB == 32 ? TB : 1;
    float ssw[4 * FB];    // per-wave sums of y^2 per token
    float ssall[8 * FB];  // this block's sums of y^2 of up to 8 heads
    __attribute__((aligned(16))) float ystash[FB * (D + 4)];  // Y of the waiting block
};

// (only transposing reads, which are never fused: no padding)
template <int TB>
struct __attribute__((aligned(16))) SmemState {
    __attribute__((aligned(16))) uint16_t kh[TB * KS];
    __attribute__((aligned(16))) uint16_t kl[TB * KS];
    __attribute__((aligned(16))) uint16_t vh[TB * KS];
    __attribute__((aligned(16))) uint16_t vl[TB * KS];
    float zpart[4 * D];
};

// Thread tid loads rows (tid>>4) + 16j, j < NJ, columns (tid&15)*8 .. +7 of
// a 16*NJ x 128 bf16 tile of one head; rows at or past nvalid read as zero.
template <int NJ>
__device__ __forceinline__ void load_tile(uint4 (&dst)[NJ], const uint16_t* __restrict__ src,
                                          int64_t t0, int nvalid, int H, int h, int tid) {
    const int col = (tid & 15) * 8;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int r = (tid >> 4) + 16 * j;
        if (r < nvalid) {
            dst[j] = *(const uint4*)(src + ((size_t)(t0 + r) * H + h) * D + col);
        } else {
            dst[j] = make_uint4(0u, 0u, 0u, 0u);
        }
    }
}

__device__ __forceinline__ void silu8(const uint4& w, float (&f)[8]) {
    f[0] = silu(bf16_lo_to_f32(w.x));
    f[1] = silu(bf16_hi_to_f32(w.x));
    f[2] = silu(bf16_lo_to_f32(w.y));
    f[3] = silu(bf16_hi_to_f32(w.y));
    f[4] = silu(bf16_lo_to_f32(w.z));
    f[5] = silu(bf16_hi_to_f32(w.z));
    f[6] = silu(bf16_lo_to_f32(w.w));
    f[7] = silu(bf16_hi_to_f32(w.w));
}

__device__ __forceinline__ void store_split8(const float (&f)[8], uint16_t* dh, uint16_t* dl) {
    uint4 hi, lo;
    split2(f[0], f[1], hi.x, lo.x);
    split2(f[2], f[3], hi.y, lo.y);
    split2(f[4], f[5], hi.z, lo.z);
    split2(f[6], f[7], hi.w, lo.w);
    *(uint4*)dh = hi;
    *(uint4*)dl = lo;
}

// phi(k) and phi(v) of the block into LDS (hi/lo); with NORM, column sums of
// phi(k) over the wave's rows into zpart[wave][col..col+7].
template <bool NORM, int NJ>
__device__ __forceinline__ void stage_kv(const uint4 (&rk)[NJ], const uint4 (&rv)[NJ],
                                         uint16_t* kh, uint16_t* kl, uint16_t* vh, uint16_t* vl,
                                         float* zpart, int tid) {
    const int col = (tid & 15) * 8;
    float zs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) zs[e] = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int r = (tid >> 4) + 16 * j;
        float f[8];
        silu8(rk[j], f);
        store_split8(f, kh + r * KS + col, kl + r * KS + col);
        if (NORM) {
#pragma unroll
            for (int e = 0; e < 8; ++e) zs[e] += f[e];
        }
        silu8(rv[j], f);
        store_split8(f, vh + r * KS + col, vl + r * KS + col);
    }
    if (NORM) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            zs[e] += __shfl_xor(zs[e], 16, 64);
            zs[e] += __shfl_xor(zs[e], 32, 64);
        }
        if ((tid & 63) < 16) {
#pragma unroll
            for (int e = 0; e < 8; ++e) zpart[(tid >> 6) * D + col + e] = zs[e];
        }
    }
}

// Operand over 32 tokens (rows of a row-major tile) for the permuted k
// order: slots {r0 + 4g + i, r0 + 16 + 4g + i}; lane (g, c) gets column c0 + c.
__device__ __forceinline__ bf16x8_t tr_operand(const uint16_t* tile, int stride, int r0, int c0,
                                               int g, int c) {
    return as_bf16x8(lds_read_tr4(tile, stride, r0 + 4 * g, c0, c),
                     lds_read_tr4(tile, stride, r0 + 16 + 4 * g, c0, c));
}

// Operand over 32 columns (head-dim features) of one row for the permuted k
// order: columns {k0 + 4g + i, k0 + 16 + 4g + i} of row `row`.  `k16` is 16
// at run time; passing it as a value keeps the two 8-byte reads separate
// (a merged 2 x 8-byte read conflicts on LDS banks, two single ones do not).
__device__ __forceinline__ bf16x8_t row_operand(const uint16_t* tile, int stride, int row, int k0,
                                                int g, int k16) {
    const uint16_t* p = tile + row * stride + k0 + 4 * g;
    return as_bf16x8(lds_read8(p), lds_read8(p + k16));
}

// State update S[dk][dv] += sum_t phi(k_t)[dk] phi(v_t)[dv] over the first
// nks*32 rows of the staged block (rows past the data are zero).
// S[dkt][dvt]: C-layout tile, lane (g, c) holds dv = 32*wave + 16*dvt + c,
// dk = 16*dkt + 4*g + i.
template <int NKS>
__device__ __forceinline__ void state_update(f32x4_t (&S)[8][2], const uint16_t* kh,
                                             const uint16_t* kl, const uint16_t* vh,
                                             const uint16_t* vl, int nks, int wave, int g, int c) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        if (ks < nks) {
            bf16x8_t Vh[2], Vl[2];
#pragma unroll
            for (int dvt = 0; dvt < 2; ++dvt) {
                const int c0 = 32 * wave + 16 * dvt;
                Vh[dvt] = tr_operand(vh, KS, 32 * ks, c0, g, c);
                Vl[dvt] = tr_operand(vl, KS, 32 * ks, c0, g, c);
            }
#pragma unroll
            for (int dkt = 0; dkt < 8; ++dkt) {
                const bf16x8_t Kh = tr_operand(kh, KS, 32 * ks, 16 * dkt, g, c);
                const bf16x8_t Kl = tr_operand(kl, KS, 32 * ks, 16 * dkt, g, c);
#pragma unroll
                for (int dvt = 0; dvt < 2; ++dvt) {
                    S[dkt][dvt] = mfma16x16x32(Kh, Vh[dvt], S[dkt][dvt]);
                    S[dkt][dvt] = mfma16x16x32(Kh, Vl[dvt], S[dkt][dvt]);
                    S[dkt][dvt] = mfma16x16x32(Kl, Vh[dvt], S[dkt][dvt]);
                }
            }
        }
    }
}

// Per-chunk state increment dS = sum_{t in chunk} phi(k_t) phi(v_t)^T (and
// dz = sum phi(k_t)), written to buf[item][h] = [dS (D*D) | dz (D)].
template <bool NORM, int TB>
__global__ __launch_bounds__(NT, 2) void k_chunk_state(const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v, ItemMap map,
                                                       int H, float* __restrict__ buf,
                                                       int64_t buf_stride) {
    using L = Tile<TB>;
    __shared__ SmemState<TB> sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c = lane & 15;
    const int h = blockIdx.y;
    Item it;
    if (!decode_item(map, blockIdx.x, it)) return;

    f32x4_t S[8][2];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) S[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float zacc = 0.f;

    const int ntiles = (it.len + TB - 1) / TB;
    uint4 rk[L::NJ], rv[L::NJ];
    load_tile<L::NJ>(rk, k, it.t0, min(TB, it.len), H, h, tid);
    load_tile<L::NJ>(rv, v, it.t0, min(TB, it.len), H, h, tid);
    for (int ti = 0; ti < ntiles; ++ti) {
        const int nvalid = min(TB, it.len - ti * TB);
        __syncthreads();
        stage_kv<NORM, L::NJ>(rk, rv, sm.kh, sm.kl, sm.vh, sm.vl, sm.zpart, tid);
        if (ti + 1 < ntiles) {
            const int64_t t1 = it.t0 + (int64_t)(ti + 1) * TB;
            const int nv1 = min(TB, it.len - (ti + 1) * TB);
            load_tile<L::NJ>(rk, k, t1, nv1, H, h, tid);
            load_tile<L::NJ>(rv, v, t1, nv1, H, h, tid);
        }
        __syncthreads();
        if (NORM && tid < D)
            zacc += (sm.zpart[tid] + sm.zpart[D + tid]) + (sm.zpart[2 * D + tid] + sm.zpart[3 * D + tid]);
        state_update<L::NKS>(S, sm.kh, sm.kl, sm.vh, sm.vl, nvalid <= 32 ? 1 : L::NKS, wave, g, c);
    }
    float* dst = buf + ((size_t)blockIdx.x * H + h) * buf_stride;
#pragma unroll
    for (int dkt = 0; dkt < 8; ++dkt)
#pragma unroll
        for (int dvt = 0; dvt < 2; ++dvt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dst[(16 * dkt + 4 * g + i) * D + 32 * wave + 16 * dvt + c] = S[dkt][dvt][i];
    if (NORM && tid < D) dst[D * D + tid] = zacc;
}

template <typename OutT> __device__ __forceinline__ void store4(OutT* p, f32x4_t v, float s);
template <> __device__ __forceinline__ void store4<float>(float* p, f32x4_t v, float s) {
    *(float4*)p = make_float4(v[0] * s, v[1] * s, v[2] * s, v[3] * s);
}
template <> __device__ __forceinline__ void store4<uint16_t>(uint16_t* p, f32x4_t v, float s) {
    uint2 u;
    u.x = pack_bf16x2(v[0] * s, v[1] * s);
    u.y = pack_bf16x2(v[2] * s, v[3] * s);
    *(uint2*)p = u;
}

// Arguments of the fused gate (RMSNorm over all H heads of a token, times
// w * sigmoid(x)), applied by the main pass when its workgroups run as
// cooperative teams of H (one per head) that exchange per-token sums of y^2.
template <typename InT>
struct GateArgs {
    const InT* x;            // [tokens, H*D]
    const float* w;          // [H*D] or nullptr
    float eps;
    uint64_t* xbuf;          // [teams][NSLOT][H][TB] (tag << 32 | sum of squares), zeroed per call
    int team;
    int spin_limit;
};
constexpr int NSLOT = 4;     // exchange slots per team: members are at most 2 blocks apart
constexpr int FUSE_HMAX = 8; // heads per token the fused gate handles (more: separate gate)

// ---- fused gate helpers ----

// After a barrier: this head's per-token sums of y^2 of the stashed block
// (summed over the 4 waves' column groups) go to the exchange buffer tagged
// with the block's sequence number.
template <int TB>
__device__ __forceinline__ void publish_ssq(SmemMain<TB>& sm, const GateArgs<uint16_t>& ga, int H,
                                            int h, uint32_t& tag) {
    ++tag;
    const int tid = threadIdx.x;
    if (tid < TB) {
        const float ss = (sm.ssw[tid] + sm.ssw[TB + tid]) + (sm.ssw[2 * TB + tid] + sm.ssw[3 * TB + tid]);
        uint64_t* slot = ga.xbuf + (((size_t)ga.team * NSLOT + (tag % NSLOT)) * H + h) * TB;
        const uint64_t word = ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(ss);
        __hip_atomic_store(slot + tid, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Keep the block's Y (acc) in LDS for the gate one block later, load its
// gate input, and put its per-wave sums of y^2 in LDS.
template <int TB>
__device__ __forceinline__ void stash_block(SmemMain<TB>& sm, const GateArgs<uint16_t>& ga,
                                            const f32x4_t (&acc)[2][Tile<TB>::NQT],
                                            uint2 (&xprev)[2][Tile<TB>::NQT], int64_t tt0,
                                            int nvalid, int H, int h, int wave, int g, int c) {
#pragma unroll
    for (int qt = 0; qt < Tile<TB>::NQT; ++qt) {
        const int row = 16 * qt + c;
        float ss = 0.f;
#pragma unroll
        for (int dvt = 0; dvt < 2; ++dvt) {
            const int col = 32 * wave + 16 * dvt + 4 * g;
            *(f32x4_t*)&sm.ystash[row * (D + 4) + col] = acc[dvt][qt];
#pragma unroll
            for (int i = 0; i < 4; ++i) ss += acc[dvt][qt][i] * acc[dvt][qt][i];
            xprev[dvt][qt] = make_uint2(0u, 0u);
            if (row < nvalid)
                xprev[dvt][qt] = *(const uint2*)(ga.x + ((size_t)(tt0 + row) * H + h) * D + col);
        }
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        if (g == 0) sm.ssw[wave * TB + row] = ss;
    }
}

// Wait for every head's sums of the stashed block, then write
// out = y / sqrt(mean over the token's H*D features of y^2 + eps) * w * sigmoid(x).
template <int TB, typename OutT>
__device__ __forceinline__ void gate_block(SmemMain<TB>& sm, const GateArgs<uint16_t>& ga,
                                           OutT* __restrict__ out,
                                           const uint2 (&xprev)[2][Tile<TB>::NQT], int64_t tprev,
                                           int nprev, int H, int h, uint32_t tag, int wave, int g,
                                           int c) {
    const int tid = threadIdx.x;
    const uint64_t* slot = ga.xbuf + ((size_t)ga.team * NSLOT + (tag % NSLOT)) * H * TB;
    for (int e = tid; e < H * TB; e += NT) {
        uint64_t word = __hip_atomic_load(slot + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int n = 0; (uint32_t)(word >> 32) != tag && n < ga.spin_limit; ++n) {
            __builtin_amdgcn_s_sleep(2);
            word = __hip_atomic_load(slot + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        sm.ssall[(e % TB) * FUSE_HMAX + e / TB] = __uint_as_float((uint32_t)word);
    }
    __syncthreads();
    const float inv_f = 1.f / (float)(H * D);
#pragma unroll
    for (int qt = 0; qt < Tile<TB>::NQT; ++qt) {
        const int row = 16 * qt + c;
        if (row >= nprev) continue;
        // heads summed in a fixed order: the result does not depend on timing
        float ss = 0.f;
        for (int hh = 0; hh < H; ++hh) ss += sm.ssall[row * FUSE_HMAX + hh];
        const float r = 1.0f / sqrtf(ss * inv_f + ga.eps);
        OutT* dst = out + ((size_t)(tprev + row) * H + h) * D + 32 * wave + 4 * g;
#pragma unroll
        for (int dvt = 0; dvt < 2; ++dvt) {
            const int col = 32 * wave + 16 * dvt + 4 * g;
            const int f = h * D + col;
            const f32x4_t yv = *(const f32x4_t*)&sm.ystash[row * (D + 4) + col];
            float xs[4] = {bf16_lo_to_f32(xprev[dvt][qt].x), bf16_hi_to_f32(xprev[dvt][qt].x),
                           bf16_lo_to_f32(xprev[dvt][qt].y), bf16_hi_to_f32(xprev[dvt][qt].y)};
            f32x4_t o;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                o[i] = yv[i] * r * (ga.w ? ga.w[f + i] : 1.f) * sigmoid(xs[i]);
            store4<OutT>(dst + 16 * dvt, o, 1.f);
        }
    }
}

// Main pass over one (chunk, head).  Starting state: prefix[item][h] if
// prefix != nullptr, else state_in/z_in of the sequence (or zeros).  When the
// chunk is a whole sequence (no prefix), the final state is written to
// state_out/z_out (if given).  Unfused: Y goes to y[t][h*D + j].  Fused: the
// gated output goes there instead, one block after Y (tag_base + block index
// numbers the exchange).  k16 must be 16.
template <bool NORM, bool FUSE, typename OutT, typename InT, int TB>
__device__ __forceinline__ void process_item(
    SmemMain<TB>& sm, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const Item& it, int item, int H, int h,
    const float* __restrict__ prefix, int64_t prefix_stride, const float* __restrict__ state_in,
    const float* __restrict__ z_in, OutT* __restrict__ y, float* state_out, float* z_out, int k16,
    const GateArgs<InT>& ga, uint32_t& tag) {
    using L = Tile<TB>;
    constexpr int PS = L::PS;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c = lane & 15;

    // P^T tiles with key tile > query tile are read by the P.V product but
    // never written: they stay zero.
    for (int i = tid; i < TB * PS / 2; i += NT) {
        ((uint32_t*)sm.ph)[i] = 0u;
        ((uint32_t*)sm.pl)[i] = 0u;
    }
    if (NORM)
        for (int i = tid; i < L::NQT * TB; i += NT) sm.denp[i] = 0.f;

    const float* s0 = nullptr;
    const float* z0 = nullptr;
    if (prefix) {
        s0 = prefix + ((size_t)item * H + h) * prefix_stride;
        z0 = s0 + D * D;
    } else {
        if (state_in) s0 = state_in + ((size_t)it.seq * H + h) * D * D;
        if (z_in) z0 = z_in + ((size_t)it.seq * H + h) * D;
    }
    f32x4_t S[8][2];
#pragma unroll
    for (int dkt = 0; dkt < 8; ++dkt)
#pragma unroll
        for (int dvt = 0; dvt < 2; ++dvt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[dkt][dvt][i] = s0 ? s0[(16 * dkt + 4 * g + i) * D + 32 * wave + 16 * dvt + c] : 0.f;
    if (NORM && tid < D) sm.z[tid] = z0 ? z0[tid] : 0.f;

    // fused gate: the previous block's Y and gate input wait here for the
    // other heads' sums of squares
    uint2 xprev[2][L::NQT];
    int64_t tprev = 0;
    int nprev = 0;

    const int ntiles = (it.len + TB - 1) / TB;
    uint4 rq[L::NJ], rk[L::NJ], rv[L::NJ];
    load_tile<L::NJ>(rq, q, it.t0, min(TB, it.len), H, h, tid);
    load_tile<L::NJ>(rk, k, it.t0, min(TB, it.len), H, h, tid);
    load_tile<L::NJ>(rv, v, it.t0, min(TB, it.len), H, h, tid);

    for (int ti = 0; ti < ntiles; ++ti) {
        const int64_t tt0 = it.t0 + (int64_t)ti * TB;
        const int nvalid = min(TB, it.len - ti * TB);
        const int nks = nvalid <= 32 ? 1 : L::NKS;  // tail pad: 32 or 64 rows
        const int nqt = 2 * nks;

        __syncthreads();  // previous block's LDS reads and z update are done
        if (FUSE && ti > 0) publish_ssq<TB>(sm, ga, H, h, tag);
        {
            const int col = (tid & 15) * 8;
#pragma unroll
            for (int j = 0; j < L::NJ; ++j) {
                const int r = (tid >> 4) + 16 * j;
                float f[8];
                silu8(rq[j], f);
                store_split8(f, sm.qh + r * QS + col, sm.ql + r * QS + col);
                if (NORM) {
                    float part = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) part += f[e] * sm.z[col + e];
                    part += __shfl_xor(part, 1, 64);
                    part += __shfl_xor(part, 2, 64);
                    part += __shfl_xor(part, 4, 64);
                    part += __shfl_xor(part, 8, 64);
                    if ((tid & 15) == 0) sm.zq[r] = part;
                }
            }
            stage_kv<NORM, L::NJ>(rk, rv, sm.kh, sm.kl, sm.vh, sm.vl, sm.zpart, tid);
        }
        if (ti + 1 < ntiles) {
            const int64_t t1 = tt0 + TB;
            const int nv1 = min(TB, it.len - (ti + 1) * TB);
            load_tile<L::NJ>(rq, q, t1, nv1, H, h, tid);
            load_tile<L::NJ>(rk, k, t1, nv1, H, h, tid);
            load_tile<L::NJ>(rv, v, t1, nv1, H, h, tid);
        }
        __syncthreads();
        if (NORM && tid < D)  // read again only after the next block's first barrier
            sm.z[tid] += (sm.zpart[tid] + sm.zpart[D + tid]) + (sm.zpart[2 * D + tid] + sm.zpart[3 * D + tid]);

        // ---- P = phi(Q) phi(K)^T on 16 x 16 tiles (query tile qt >= key tile kt),
        //      causal mask, stored transposed as P^T[key][query] ----
        {
            const int ntau = nks == 2 ? 10 : 3;
            for (int tau = wave; tau < ntau; tau += 4) {
                const int qt = tau >= 6 ? 3 : tau >= 3 ? 2 : tau >= 1 ? 1 : 0;
                const int kt = tau - qt * (qt + 1) / 2;
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const bf16x8_t ah = row_operand(sm.qh, QS, 16 * qt + c, 32 * s, g, k16);
                    const bf16x8_t al = row_operand(sm.ql, QS, 16 * qt + c, 32 * s, g, k16);
                    const bf16x8_t bh = row_operand(sm.kh, KS, 16 * kt + c, 32 * s, g, k16);
                    const bf16x8_t bl = row_operand(sm.kl, KS, 16 * kt + c, 32 * s, g, k16);
                    acc = mfma16x16x32(ah, bh, acc);
                    acc = mfma16x16x32(ah, bl, acc);
                    acc = mfma16x16x32(al, bh, acc);
                }
                // acc[i]: query 16qt + 4g + i, key 16kt + c; keep key <= query
                if (kt == qt) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (c > 4 * g + i) acc[i] = 0.f;
                }
                uint2 pkh, pkl;
                split2(acc[0], acc[1], pkh.x, pkl.x);
                split2(acc[2], acc[3], pkh.y, pkl.y);
                const int po = (16 * kt + c) * PS + 16 * qt + 4 * g;
                *(uint2*)&sm.ph[po] = pkh;
                *(uint2*)&sm.pl[po] = pkl;
                if (NORM) {
                    // row sums over this tile's 16 keys (the 16 lanes of a group)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float rs = acc[i];
                        rs += __shfl_xor(rs, 1, 64);
                        rs += __shfl_xor(rs, 2, 64);
                        rs += __shfl_xor(rs, 4, 64);
                        rs += __shfl_xor(rs, 8, 64);
                        if (c == 0) sm.denp[kt * TB + 16 * qt + 4 * g + i] = rs;
                    }
                }
            }
        }
        __syncthreads();

        // ---- Y^T = V^T P^T (intra) + S^T Q^T (inter), this wave's 32 columns ----
        f32x4_t acc[2][L::NQT];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < L::NQT; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // intra: key steps outer, both value tiles per P^T operand
#pragma unroll
        for (int ks = 0; ks < L::NKS; ++ks) {
            if (ks < nks) {
                bf16x8_t Ah[2], Al[2];
#pragma unroll
                for (int dvt = 0; dvt < 2; ++dvt) {
                    const int c0 = 32 * wave + 16 * dvt;
                    Ah[dvt] = tr_operand(sm.vh, KS, 32 * ks, c0, g, c);
                    Al[dvt] = tr_operand(sm.vl, KS, 32 * ks, c0, g, c);
                }
#pragma unroll
                for (int qt = 0; qt < L::NQT; ++qt) {
                    if (qt < nqt && (ks == 0 || qt >= 2)) {
                        const bf16x8_t bh = tr_operand(sm.ph, PS, 32 * ks, 16 * qt, g, c);
                        const bf16x8_t bl = tr_operand(sm.pl, PS, 32 * ks, 16 * qt, g, c);
#pragma unroll
                        for (int dvt = 0; dvt < 2; ++dvt) {
                            acc[dvt][qt] = mfma16x16x32(Ah[dvt], bh, acc[dvt][qt]);
                            acc[dvt][qt] = mfma16x16x32(Ah[dvt], bl, acc[dvt][qt]);
                            acc[dvt][qt] = mfma16x16x32(Al[dvt], bh, acc[dvt][qt]);
                        }
                    }
                }
            }
        }
        // inter: head-dim steps outer; the state's split for both value tiles,
        // then each Q^T operand feeds both
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8_t Ah[2], Al[2];
#pragma unroll
            for (int dvt = 0; dvt < 2; ++dvt) {
                uint4 ah, al;
                split2(S[2 * s][dvt][0], S[2 * s][dvt][1], ah.x, al.x);
                split2(S[2 * s][dvt][2], S[2 * s][dvt][3], ah.y, al.y);
                split2(S[2 * s + 1][dvt][0], S[2 * s + 1][dvt][1], ah.z, al.z);
                split2(S[2 * s + 1][dvt][2], S[2 * s + 1][dvt][3], ah.w, al.w);
                Ah[dvt] = as_bf16x8(ah);
                Al[dvt] = as_bf16x8(al);
            }
#pragma unroll
            for (int qt = 0; qt < L::NQT; ++qt) {
                if (qt < nqt) {
                    const bf16x8_t Bh = row_operand(sm.qh, QS, 16 * qt + c, 32 * s, g, k16);
                    const bf16x8_t Bl = row_operand(sm.ql, QS, 16 * qt + c, 32 * s, g, k16);
#pragma unroll
                    for (int dvt = 0; dvt < 2; ++dvt) {
                        acc[dvt][qt] = mfma16x16x32(Ah[dvt], Bh, acc[dvt][qt]);
                        acc[dvt][qt] = mfma16x16x32(Ah[dvt], Bl, acc[dvt][qt]);
                        acc[dvt][qt] = mfma16x16x32(Al[dvt], Bh, acc[dvt][qt]);
                    }
                }
            }
        }
        // acc[dvt][qt][i]: query 16qt + c, feature 32*wave + 16*dvt + 4g + i
        if (NORM) {
#pragma unroll
            for (int qt = 0; qt < L::NQT; ++qt) {
                const int row = 16 * qt + c;
                float den = sm.zq[row];
                for (int kt = 0; kt <= qt; ++kt) den += sm.denp[kt * TB + row];
                const float sc = 1.f / den;
#pragma unroll
                for (int dvt = 0; dvt < 2; ++dvt) acc[dvt][qt] *= sc;
            }
        }
        if (!FUSE) {
#pragma unroll
            for (int qt = 0; qt < L::NQT; ++qt) {
                const int row = 16 * qt + c;
                if (qt < nqt && row < nvalid) {
                    OutT* dst = y + ((size_t)(tt0 + row) * H + h) * D + 32 * wave + 4 * g;
#pragma unroll
                    for (int dvt = 0; dvt < 2; ++dvt) store4<OutT>(dst + 16 * dvt, acc[dvt][qt], 1.f);
                }
            }
        } else {
            if (ti > 0) gate_block<TB>(sm, ga, y, xprev, tprev, nprev, H, h, tag, wave, g, c);
            __syncthreads();  // the stash is read by other waves' gate above
            stash_block<TB>(sm, ga, acc, xprev, tt0, nvalid, H, h, wave, g, c);
            tprev = tt0;
            nprev = nvalid;
        }

        // ---- S += phi(K)^T phi(V) ----
        state_update<L::NKS>(S, sm.kh, sm.kl, sm.vh, sm.vl, nks, wave, g, c);
    }
    if (FUSE) {
        __syncthreads();
        publish_ssq<TB>(sm, ga, H, h, tag);
        gate_block<TB>(sm, ga, y, xprev, tprev, nprev, H, h, tag, wave, g, c);
    }

    if (!prefix) {
        if (state_out) {
            float* dst = state_out + ((size_t)it.seq * H + h) * D * D;
#pragma unroll
            for (int dkt = 0; dkt < 8; ++dkt)
#pragma unroll
                for (int dvt = 0; dvt < 2; ++dvt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        dst[(16 * dkt + 4 * g + i) * D + 32 * wave + 16 * dvt + c] = S[dkt][dvt][i];
        }
        if (NORM && z_out) {
            __syncthreads();
            if (tid < D) z_out[((size_t)it.seq * H + h) * D + tid] = sm.z[tid];
        }
    }
    __syncthreads();  // the next item reuses the LDS
}

// Unfused main pass: one workgroup per (chunk = blockIdx.x, head = blockIdx.y).
template <bool NORM, typename OutT, int TB>
__global__ __launch_bounds__(NT, Tile<TB>::WG_PER_CU) void k_prefill_main(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    ItemMap map, int H, const float* __restrict__ prefix, int64_t prefix_stride,
    const float* __restrict__ state_in, const float* __restrict__ z_in, OutT* __restrict__ y,
    float* state_out, float* z_out, int k16) {
    __shared__ SmemMain<TB> sm;
    Item it;
    if (!decode_item(map, blockIdx.x, it)) return;
    GateArgs<uint16_t> ga{};
    uint32_t tag = 0;
    process_item<NORM, false, OutT, uint16_t, TB>(sm, q, k, v, it, blockIdx.x, H, blockIdx.y,
                                                   prefix, prefix_stride, state_in, z_in, y,
                                                   state_out, z_out, k16, ga, tag);
}

// Fused main pass + gate, one workgroup per (chunk = blockIdx.x / H, head =
// blockIdx.x % H).  Launched cooperatively: every workgroup is resident, so
// the H heads of a chunk -- a team -- run together and their per-token sums
// of y^2 meet in the exchange buffer.  Every wait is bounded.
template <bool NORM, typename OutT, int TB>
__global__ __launch_bounds__(NT, Tile<TB>::WG_PER_CU) void k_prefill_fused(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    ItemMap map, int H, const float* __restrict__ prefix, int64_t prefix_stride,
    const float* __restrict__ state_in, const float* __restrict__ z_in, OutT* __restrict__ out,
    float* state_out, float* z_out, int k16, const uint16_t* __restrict__ x,
    const float* __restrict__ w, float eps, uint64_t* xbuf, int spin_limit) {
    __shared__ SmemMain<TB> sm;
    const int item = blockIdx.x / H, h = blockIdx.x - item * H;
    Item it;
    if (!decode_item(map, item, it)) return;  // the whole team returns together
    GateArgs<uint16_t> ga{x, w, eps, xbuf, item, spin_limit};
    uint32_t tag = 0;
    process_item<NORM, true, OutT, uint16_t, TB>(sm, q, k, v, it, item, H, h, prefix,
                                                  prefix_stride, state_in, z_in, out, state_out,
                                                  z_out, k16, ga, tag);
}

}  // namespace mf
}  // namespace la
