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
//    workgroup is 79 KiB (60 KiB of q, k, v and P^T tiles, the rest the fused
//    gate's stash of Y and sums) and two workgroups share a CU, so one's
//    SiLU/split VALU work overlaps the other's matrix-core work; wave w owns value columns
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

#include <type_traits>

#include "la_device.h"
#include "la_items.h"

namespace la {
namespace mf {

constexpr int D = 128;   // head dim
constexpr int NT = 256;  // threads per workgroup
// LDS row strides (bf16 elements).  Q is read only along rows, two 8-byte
// pieces per lane that the compiler merges into one ds_read2_b64: at a
// stride of 132 (264 bytes) such pairs hit 64 distinct banks, at 136 or 144
// they conflict (measured).  K and V are read by transposing reads, which
// need 144; their row reads (K in P) stay single 8-byte reads.
constexpr int QS = 132;  // Q tile
constexpr int KS = 144;  // K and V tiles
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
    float ssw[4 * FB];  // per-wave sums of y^2 per token
    float ssum[FB];     // all heads' sums of y^2 per token
    __attribute__((aligned(16))) float wgate[TB == 32 ? D : 4];  // this head's RMSNorm weights
    __attribute__((aligned(16))) float ystash[FB * (D + 4)];  // Y of the block awaiting its gate
};

// Chunk-state pass: two 32-token buffers (only transposing reads, which are
// never fused: no padding).
struct __attribute__((aligned(16))) SmemState {
    static constexpr int TB = 32;
    __attribute__((aligned(16))) uint16_t kh[2][TB * KS];
    __attribute__((aligned(16))) uint16_t kl[2][TB * KS];
    __attribute__((aligned(16))) uint16_t vh[2][TB * KS];
    __attribute__((aligned(16))) uint16_t vl[2][TB * KS];
    float zpart[2][4 * D];
};

// Thread tid loads rows (tid>>4) + 16j, j < NJ, columns (tid&15)*8 .. +7 of
// a 16*NJ x 128 bf16 tile of one head; rows at or past nvalid read as zero.
// `blk` points at the tile's first row (same for the whole workgroup) and
// `rs` is the row stride in elements (H*D).
template <int NJ>
__device__ __forceinline__ void load_tile(uint4 (&dst)[NJ], const uint16_t* __restrict__ blk,
                                          uint32_t rs, int nvalid, int tid) {
    const uint32_t off = (uint32_t)(tid >> 4) * rs + (uint32_t)(tid & 15) * 8;
    if (nvalid >= 16 * NJ) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) dst[j] = *(const uint4*)(blk + off + (uint32_t)(16 * j) * rs);
    } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int r = (tid >> 4) + 16 * j;
            dst[j] = r < nvalid ? *(const uint4*)(blk + off + (uint32_t)(16 * j) * rs)
                                : make_uint4(0u, 0u, 0u, 0u);
        }
    }
}

// First element of token t, head h of a [tokens, H, D] tensor.
__device__ __forceinline__ const uint16_t* head_row(const uint16_t* p, int64_t t, int H, int h) {
    return p + ((size_t)t * H + h) * D;
}

// Buffer resource over the rows [0, nvalid) of one head's tile starting at
// `blk` (row stride rs elements): loads past the last valid row return zero
// with no memory access (nvalid <= 0: every load does).  A tile has at most
// 64 rows, so the range is capped there (it then fits the 32-bit size field
// for any row stride the library accepts).  Word 3 is the gfx9 raw-buffer
// configuration (32-bit data format, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* blk, uint32_t rs,
                                                            int nvalid) {
    nvalid = min(nvalid, 64);
    const int32_t bytes = nvalid > 0 ? (int32_t)((uint32_t)(nvalid - 1) * rs * 2u + 2u * D) : 0;
    return __builtin_amdgcn_make_buffer_rsrc((void*)blk, (short)0, bytes, 0x00020000);
}

// Buffer resource over `nrows` rows of `width_bytes` each, `row_bytes` apart,
// from `base`: accesses past the last row are dropped (stores) or read zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, uint32_t row_bytes,
                                                            uint32_t width_bytes, int nrows) {
    const int32_t bytes = nrows > 0 ? (int32_t)((uint32_t)(nrows - 1) * row_bytes + width_bytes) : 0;
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, 0x00020000);
}

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

// Four outputs at element offset `off` through a rows_rsrc (dropped past its rows).
template <typename OutT>
__device__ __forceinline__ void store4_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4_t v);
template <>
__device__ __forceinline__ void store4_buf<float>(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4_t v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off * 4u, 0, 0);
}
template <>
__device__ __forceinline__ void store4_buf<uint16_t>(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4_t v) {
    const u32x2_t u = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    __builtin_amdgcn_raw_buffer_store_b64(u, r, off * 2u, 0, 0);
}

// load_tile through a tile_rsrc: no branches, zeros past the valid rows.
template <int NJ>
__device__ __forceinline__ void load_tile_buf(uint4 (&dst)[NJ], __amdgpu_buffer_rsrc_t rsrc,
                                              uint32_t rs, int tid) {
    const uint32_t off = ((uint32_t)(tid >> 4) * rs + (uint32_t)(tid & 15) * 8) * 2u;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const auto w = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off + (uint32_t)(16 * j) * rs * 2u, 0, 0);
        dst[j] = __builtin_bit_cast(uint4, w);
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

// Eight bf16 values as fp32 (no feature map: the inputs are features already).
__device__ __forceinline__ void unpack8(const uint4& w, float (&f)[8]) {
    f[0] = bf16_lo_to_f32(w.x);
    f[1] = bf16_hi_to_f32(w.x);
    f[2] = bf16_lo_to_f32(w.y);
    f[3] = bf16_hi_to_f32(w.y);
    f[4] = bf16_lo_to_f32(w.z);
    f[5] = bf16_hi_to_f32(w.z);
    f[6] = bf16_lo_to_f32(w.w);
    f[7] = bf16_hi_to_f32(w.w);
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

// The same into rows that are only 8-byte aligned (the Q tile).
__device__ __forceinline__ void store_split8_a8(const float (&f)[8], uint16_t* dh, uint16_t* dl) {
    uint2 h0, h1, l0, l1;
    split2(f[0], f[1], h0.x, l0.x);
    split2(f[2], f[3], h0.y, l0.y);
    split2(f[4], f[5], h1.x, l1.x);
    split2(f[6], f[7], h1.y, l1.y);
    *(uint2*)dh = h0;
    *(uint2*)(dh + 4) = h1;
    *(uint2*)dl = l0;
    *(uint2*)(dl + 4) = l1;
}

// phi(k) and phi(v) of the block into LDS (hi/lo); with NORM, column sums of
// phi(k) over the wave's rows into zpart[wave][col..col+7].  FEAT: k and v
// are feature vectors already, exact in bf16: stored as they are, no low part.
template <bool NORM, int NJ, bool FEAT = false>
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
        if constexpr (FEAT) {
            *(uint4*)(kh + r * KS + col) = rk[j];
            *(uint4*)(vh + r * KS + col) = rv[j];
            if (NORM) unpack8(rk[j], f);
        } else {
            silu8(rk[j], f);
            store_split8(f, kh + r * KS + col, kl + r * KS + col);
        }
        if (NORM) {
#pragma unroll
            for (int e = 0; e < 8; ++e) zs[e] += f[e];
        }
        if constexpr (!FEAT) {
            silu8(rv[j], f);
            store_split8(f, vh + r * KS + col, vl + r * KS + col);
        }
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
// order: columns {k0 + 4g + i, k0 + 16 + 4g + i} of row `row`.  With k16 a
// literal 16 the compiler merges the two 8-byte reads into one ds_read2_b64
// (conflict-free at the Q stride); passed as a run-time value (16), it keeps
// them separate, which the K stride needs.
__device__ __forceinline__ bf16x8_t row_operand(const uint16_t* tile, int stride, int row, int k0,
                                                int g, int k16) {
    const uint16_t* p = tile + row * stride + k0 + 4 * g;
    return as_bf16x8(lds_read8(p), lds_read8(p + k16));
}

// State update S[dk][dv] += sum_t phi(k_t)[dk] phi(v_t)[dv] over the first
// nks*32 rows of the staged block (rows past the data are zero).
// S[dkt][dvt]: C-layout tile, lane (g, c) holds dv = 32*wave + 16*dvt + c,
// dk = 16*dkt + 4*g + i.
template <int NKS, bool FEAT = false>
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
                if constexpr (!FEAT) Vl[dvt] = tr_operand(vl, KS, 32 * ks, c0, g, c);
            }
#pragma unroll
            for (int dkt = 0; dkt < 8; ++dkt) {
                const bf16x8_t Kh = tr_operand(kh, KS, 32 * ks, 16 * dkt, g, c);
                if constexpr (FEAT) {
                    // bf16-exact features: one product is exact
#pragma unroll
                    for (int dvt = 0; dvt < 2; ++dvt)
                        S[dkt][dvt] = mfma16x16x32(Kh, Vh[dvt], S[dkt][dvt]);
                } else {
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
}

// Per-chunk state increment dS = sum_{t in chunk} phi(k_t) phi(v_t)^T (and
// dz = sum phi(k_t)), written to buf[item][h] = [dS (D*D) | dz (D)].  The
// last chunk of a sequence is skipped: no later chunk starts from it, and the
// main pass writes the sequence's final state.
// Software-pipelined over 32-token blocks with two LDS buffers: in step n
// the workgroup stages block n+1 (SiLU + split, vector ALU) into one buffer
// while the state update of block n (matrix cores) reads the other, with
// one barrier per step; raw k, v are loaded two blocks ahead.
template <bool NORM, bool FEAT = false>
__global__ __launch_bounds__(NT, 2) void k_chunk_state(const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v, ItemMap map,
                                                       int H, float* __restrict__ buf,
                                                       int64_t buf_stride) {
    constexpr int TB = SmemState::TB;
    using L = Tile<TB>;
    __shared__ SmemState sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c = lane & 15;
    (void)lane;
    const int h = blockIdx.y;
    Item it;
    if (!decode_item(map, blockIdx.x, it) || it.last) return;

    f32x4_t S[8][2];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) S[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float zacc = 0.f;

    const int ntiles = (it.len + TB - 1) / TB;
    const uint32_t rs = (uint32_t)H * D;
    const uint16_t* kb = head_row(k, it.t0, H, h);
    const uint16_t* vb = head_row(v, it.t0, H, h);
    uint4 rk[L::NJ], rv[L::NJ];
    // block 0 staged, block 1 in registers
    load_tile_buf<L::NJ>(rk, tile_rsrc(kb, rs, it.len), rs, tid);
    load_tile_buf<L::NJ>(rv, tile_rsrc(vb, rs, it.len), rs, tid);
    stage_kv<NORM, L::NJ, FEAT>(rk, rv, sm.kh[0], sm.kl[0], sm.vh[0], sm.vl[0], sm.zpart[0], tid);
    kb += (size_t)TB * rs;
    vb += (size_t)TB * rs;
    load_tile_buf<L::NJ>(rk, tile_rsrc(kb, rs, it.len - TB), rs, tid);
    load_tile_buf<L::NJ>(rv, tile_rsrc(vb, rs, it.len - TB), rs, tid);
    __syncthreads();
    // one step: state update of block ti from buffer CUR, staging of block
    // ti+1 into the other buffer, loads of block ti+2 (the buffers are
    // compile-time distinct, so the update's reads and the staging's writes
    // may interleave)
    auto step = [&](auto cur_tag, int ti) {
        constexpr int CUR = decltype(cur_tag)::value;
        if (NORM && tid < D)
            zacc += (sm.zpart[CUR][tid] + sm.zpart[CUR][D + tid]) +
                    (sm.zpart[CUR][2 * D + tid] + sm.zpart[CUR][3 * D + tid]);
        uint4 nk[L::NJ], nv[L::NJ];
        kb += (size_t)TB * rs;
        vb += (size_t)TB * rs;
        const int n2 = it.len - (ti + 2) * TB;
        load_tile_buf<L::NJ>(nk, tile_rsrc(kb, rs, n2), rs, tid);
        load_tile_buf<L::NJ>(nv, tile_rsrc(vb, rs, n2), rs, tid);
        state_update<1, FEAT>(S, sm.kh[CUR], sm.kl[CUR], sm.vh[CUR], sm.vl[CUR], 1, wave, g, c);
        stage_kv<NORM, L::NJ, FEAT>(rk, rv, sm.kh[CUR ^ 1], sm.kl[CUR ^ 1], sm.vh[CUR ^ 1],
                              sm.vl[CUR ^ 1], sm.zpart[CUR ^ 1], tid);
#pragma unroll
        for (int j = 0; j < L::NJ; ++j) {
            rk[j] = nk[j];
            rv[j] = nv[j];
        }
        __syncthreads();
    };
    for (int ti = 0; ti < ntiles; ti += 2) {
        step(std::integral_constant<int, 0>{}, ti);
        if (ti + 1 == ntiles) break;
        step(std::integral_constant<int, 1>{}, ti + 1);
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

// The same increment with one staging buffer (39 KB of LDS, at most 128
// VGPRs): four workgroups per CU, whose interleaving hides the latency that
// the two-buffer pipeline above hides inside one workgroup.  Per 32-token
// block: stage (SiLU + split), load the next block, barrier, state update,
// barrier.  Used for plans with twice as many chunks as resident slots of the
// two-buffer kernel.
struct SmemState1 {
    static constexpr int TB = 32;
    __attribute__((aligned(16))) uint16_t kh[TB * KS];
    __attribute__((aligned(16))) uint16_t kl[TB * KS];
    __attribute__((aligned(16))) uint16_t vh[TB * KS];
    __attribute__((aligned(16))) uint16_t vl[TB * KS];
    float zpart[4 * D];
};

template <bool NORM, bool FEAT = false>
__global__ __launch_bounds__(NT, 4) void k_chunk_state1(const uint16_t* __restrict__ k,
                                                        const uint16_t* __restrict__ v, ItemMap map,
                                                        int H, float* __restrict__ buf,
                                                        int64_t buf_stride) {
    constexpr int TB = SmemState1::TB;
    using L = Tile<TB>;
    __shared__ SmemState1 sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c = lane & 15;
    const int h = blockIdx.y;
    Item it;
    if (!decode_item(map, blockIdx.x, it) || it.last) return;

    f32x4_t S[8][2];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) S[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float zacc = 0.f;

    const int ntiles = (it.len + TB - 1) / TB;
    const uint32_t rs = (uint32_t)H * D;
    const uint16_t* kb = head_row(k, it.t0, H, h);
    const uint16_t* vb = head_row(v, it.t0, H, h);
    uint4 rk[L::NJ], rv[L::NJ];
    load_tile_buf<L::NJ>(rk, tile_rsrc(kb, rs, it.len), rs, tid);
    load_tile_buf<L::NJ>(rv, tile_rsrc(vb, rs, it.len), rs, tid);
    for (int ti = 0; ti < ntiles; ++ti) {
        stage_kv<NORM, L::NJ, FEAT>(rk, rv, sm.kh, sm.kl, sm.vh, sm.vl, sm.zpart, tid);
        kb += (size_t)TB * rs;
        vb += (size_t)TB * rs;
        const int n1 = it.len - (ti + 1) * TB;  // <= 0 past the last block: zeros, never staged
        load_tile_buf<L::NJ>(rk, tile_rsrc(kb, rs, n1), rs, tid);
        load_tile_buf<L::NJ>(rv, tile_rsrc(vb, rs, n1), rs, tid);
        __syncthreads();
        if (NORM && tid < D)
            zacc += (sm.zpart[tid] + sm.zpart[D + tid]) + (sm.zpart[2 * D + tid] + sm.zpart[3 * D + tid]);
        state_update<1, FEAT>(S, sm.kh, sm.kl, sm.vh, sm.vl, 1, wave, g, c);
        __syncthreads();
    }
    (void)lane;
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
    int spin_limit;          // retries per wait; < 0: every wait gives up at once
    uint32_t* status;        // set to 1 when a wait gives up (zeroed per call)
};
constexpr int NSLOT = 4;     // exchange slots per team (2 suffice: see publish order)
constexpr int FUSE_HMAX = 8; // heads per token the fused gate handles (more: separate gate)

// ---- fused gate helpers ----

// Keep the block's Y in LDS until its gate one block later (each wave
// writes, and later reads, only its own 32 columns), put its per-wave sums
// of y^2 per token in ssw[wave][row], and load its gate input (xrs: the
// block's rows of x, zero past the valid ones).
template <int TB>
__device__ __forceinline__ void stash_block(SmemMain<TB>& sm, const f32x4_t (&acc)[2][Tile<TB>::NQT],
                                            uint2 (&xr)[2][Tile<TB>::NQT],
                                            __amdgpu_buffer_rsrc_t xrs, uint32_t rs, int wave, int g,
                                            int c) {
#pragma unroll
    for (int qt = 0; qt < Tile<TB>::NQT; ++qt) {
        const int row = 16 * qt + c;
        float ss = 0.f;
#pragma unroll
        for (int dvt = 0; dvt < 2; ++dvt) {
            *(f32x4_t*)&sm.ystash[row * (D + 4) + 32 * wave + 16 * dvt + 4 * g] = acc[dvt][qt];
#pragma unroll
            for (int i = 0; i < 4; ++i) ss += acc[dvt][qt][i] * acc[dvt][qt][i];
            const uint32_t off = ((uint32_t)row * rs + 32 * wave + 16 * dvt + 4 * g) * 2u;
            xr[dvt][qt] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(xrs, off, 0, 0));
        }
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        sm.ssw[wave * TB + row] = ss;  // the 4 lane groups hold the same sum: no branch
    }
}

// After gather_finish and a barrier: out = y / sqrt(mean over the token's H*D
// features of y^2 + eps) * w * sigmoid(x) for the stashed block; `ors`
// covers its valid output rows (stores past them are dropped), so the code
// has no branches.
template <int TB, typename OutT>
__device__ __forceinline__ void gate_block(const SmemMain<TB>& sm, __amdgpu_buffer_rsrc_t ors,
                                           const uint2 (&xr)[2][Tile<TB>::NQT], float inv_f, float eps,
                                           uint32_t rs, int wave, int g, int c) {
#pragma unroll
    for (int qt = 0; qt < Tile<TB>::NQT; ++qt) {
        const int row = 16 * qt + c;
        const float r = rsqrtf(sm.ssum[row] * inv_f + eps);
#pragma unroll
        for (int dvt = 0; dvt < 2; ++dvt) {
            const int col = 32 * wave + 16 * dvt + 4 * g;
            const f32x4_t yv = *(const f32x4_t*)&sm.ystash[row * (D + 4) + col];
            const f32x4_t wv = *(const f32x4_t*)&sm.wgate[col];
            const float xs[4] = {bf16_lo_to_f32(xr[dvt][qt].x), bf16_hi_to_f32(xr[dvt][qt].x),
                                 bf16_lo_to_f32(xr[dvt][qt].y), bf16_hi_to_f32(xr[dvt][qt].y)};
            f32x4_t o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = yv[i] * r * wv[i] * sigmoid(xs[i]);
            store4_buf<OutT>(ors, (uint32_t)row * rs + col, o);
        }
    }
}

// After a barrier: the head's per-token sums (the 4 waves' column groups
// added) go to its slot of the exchange buffer, tagged with the block's
// sequence number.  Threads of wave 0 only.
template <int TB>
__device__ __forceinline__ void publish_ssq(const SmemMain<TB>& sm, const GateArgs<uint16_t>& ga,
                                            int H, int h, uint32_t tag) {
    const int tid = threadIdx.x;
    if (tid < TB) {
        const float ss = (sm.ssw[tid] + sm.ssw[TB + tid]) + (sm.ssw[2 * TB + tid] + sm.ssw[3 * TB + tid]);
        uint64_t* slot = ga.xbuf + (((size_t)ga.team * NSLOT + (tag % NSLOT)) * H + h) * TB;
        const uint64_t word = ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(ss);
        __hip_atomic_store(slot + tid, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Wave 0, in two steps: gather_issue starts the loads of the team's words
// for block `tag` (lane l: words l + 64j, i.e. head l/32 + 2j, token l%32);
// gather_finish, later, re-reads (bounded) any word whose tag is not yet
// current, then ssum[token] = sum over heads.  The heads are added in a
// fixed order, so the sum does not depend on timing.
template <int TB>
__device__ __forceinline__ void gather_issue(const GateArgs<uint16_t>& ga, int H, uint32_t tag,
                                             int lane, uint64_t (&word)[4]) {
    static_assert(TB == 32, "the fused gate runs on 32-token blocks");
    const uint64_t* slot = ga.xbuf + ((size_t)ga.team * NSLOT + (tag % NSLOT)) * H * TB;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
        word[j] = e < H * TB ? __hip_atomic_load(slot + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                             : (uint64_t)tag << 32;
    }
}

// A wait that gives up (spin_limit retries, or at once when spin_limit < 0)
// never gates with a word it could not verify: the token's sum becomes NaN,
// so its gated outputs are NaN, and the call's status word is set.  (A word
// with the current tag is always this block's: an older block in the same
// slot carries a tag NSLOT * n smaller.)
template <int TB>
__device__ __forceinline__ void gather_finish(SmemMain<TB>& sm, const GateArgs<uint16_t>& ga,
                                              int H, uint32_t tag, int lane, uint64_t (&word)[4]) {
    const uint64_t* slot = ga.xbuf + ((size_t)ga.team * NSLOT + (tag % NSLOT)) * H * TB;
    bool ready = false;
    for (int n = 0;; ++n) {
        ready = ga.spin_limit >= 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) ready = ready && (word[j] >> 32) == (uint64_t)tag;
        if (ready || n >= ga.spin_limit) break;
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = lane + 64 * j;
            if ((word[j] >> 32) != (uint64_t)tag)
                word[j] = __hip_atomic_load(slot + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    float ss = (__uint_as_float((uint32_t)word[0]) + __uint_as_float((uint32_t)word[1])) +
               (__uint_as_float((uint32_t)word[2]) + __uint_as_float((uint32_t)word[3]));
    if (!ready) {
        ss = __builtin_nanf("");
        __hip_atomic_store(ga.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    ss += __shfl_xor(ss, 32, 64);
    if (lane < TB) sm.ssum[lane] = ss;
}

// phi(q) of the block into the Q tile (hi/lo); with NORM zq[row] = phi(q_row) . z.
template <bool NORM, int NJ, typename SM, bool FEAT = false>
__device__ __forceinline__ void stage_q(SM& sm, const uint4 (&rq)[NJ], int tid) {
    const int col = (tid & 15) * 8;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int r = (tid >> 4) + 16 * j;
        float f[8];
        if constexpr (FEAT) {
            *(uint2*)(sm.qh + r * QS + col) = make_uint2(rq[j].x, rq[j].y);
            *(uint2*)(sm.qh + r * QS + col + 4) = make_uint2(rq[j].z, rq[j].w);
            if (NORM) unpack8(rq[j], f);
        } else {
            silu8(rq[j], f);
            store_split8_a8(f, sm.qh + r * QS + col, sm.ql + r * QS + col);
        }
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
}

// Main pass over one (chunk, head).  Starting state: prefix[item][h] if
// prefix != nullptr, else state_in/z_in of the sequence (or zeros).  After the
// last chunk of a sequence the final state is written to state_out/z_out (if
// given).  Unfused: Y goes to y[t][h*D + j].  Fused: the
// gated output goes there instead; the heads of the chunk exchange each
// block's per-token sums of y^2 (tag = block number + 1).  k16 must be 16.
template <bool NORM, bool FUSE, typename OutT, typename InT, int TB, bool FEAT>
__device__ __forceinline__ void process_item(
    SmemMain<TB>& sm, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const Item& it, int item, int H, int h,
    const float* __restrict__ prefix, int64_t prefix_stride, const float* __restrict__ state_in,
    const float* __restrict__ z_in, OutT* __restrict__ y, float* state_out, float* z_out, int k16,
    const GateArgs<InT>& ga) {
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
        if (state_in && it.row >= 0) s0 = state_in + ((size_t)it.row * H + h) * D * D;
        if (z_in && it.row >= 0) z0 = z_in + ((size_t)it.row * H + h) * D;
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

    // fused gate: the gate of block n runs one block later, when the other heads' sums of
    // y^2 for it have had a block's time to arrive
    uint2 xr[2][L::NQT];  // gate input of the stashed block
    const uint16_t* xb = nullptr;  // x rows of the current block (this head)
    OutT* ob = y;                  // output rows of the stashed block
    int nprev = 0;
    float inv_f = 0.f;
    if constexpr (FUSE) {
        if (tid < D) sm.wgate[tid] = ga.w ? ga.w[h * D + tid] : 1.f;  // read after the first barrier
        xb = ga.x + ((size_t)it.t0 * H + h) * D;
        inv_f = 1.f / (float)(H * D);
    }

    const int ntiles = (it.len + TB - 1) / TB;
    const uint32_t rs = (uint32_t)H * D;
    const uint16_t* qb = head_row(q, it.t0, H, h);
    const uint16_t* kb = head_row(k, it.t0, H, h);
    const uint16_t* vb = head_row(v, it.t0, H, h);
    uint4 rq[L::NJ], rk[L::NJ], rv[L::NJ];
    const int nv0 = min(TB, it.len);
    load_tile_buf<L::NJ>(rq, tile_rsrc(qb, rs, nv0), rs, tid);
    load_tile_buf<L::NJ>(rk, tile_rsrc(kb, rs, nv0), rs, tid);
    load_tile_buf<L::NJ>(rv, tile_rsrc(vb, rs, nv0), rs, tid);
    __syncthreads();  // z (normalised mode) is set
    // the Q tile of block n is staged at the end of block n-1 (here, block 0)
    stage_q<NORM, L::NJ, SmemMain<TB>, FEAT>(sm, rq, tid);

    for (int ti = 0; ti < ntiles; ++ti) {
        const int64_t tt0 = it.t0 + (int64_t)ti * TB;
        const int nvalid = min(TB, it.len - ti * TB);
        const int nks = nvalid <= 32 ? 1 : L::NKS;  // tail pad: 32 or 64 rows
        const int nqt = 2 * nks;

        __syncthreads();  // previous block's LDS reads and z update are done
        if constexpr (FUSE) {
            if (ti > 0) publish_ssq<TB>(sm, ga, H, h, (uint32_t)ti);
        }
        stage_kv<NORM, L::NJ, FEAT>(rk, rv, sm.kh, sm.kl, sm.vh, sm.vl, sm.zpart, tid);
        if (ti + 1 < ntiles) {
            const int nv1 = min(TB, it.len - (ti + 1) * TB);
            qb += (size_t)TB * rs;
            kb += (size_t)TB * rs;
            vb += (size_t)TB * rs;
            load_tile_buf<L::NJ>(rq, tile_rsrc(qb, rs, nv1), rs, tid);
            load_tile_buf<L::NJ>(rk, tile_rsrc(kb, rs, nv1), rs, tid);
            load_tile_buf<L::NJ>(rv, tile_rsrc(vb, rs, nv1), rs, tid);
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
                // three independent accumulator chains (hi.hi, hi.lo, lo.hi)
                f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const bf16x8_t ah = row_operand(sm.qh, QS, 16 * qt + c, 32 * s, g, 16);
                    // run-time column steps: no merged K reads (they conflict at KS)
                    const bf16x8_t bh = row_operand(sm.kh, KS, 16 * kt + c, 2 * k16 * s, g, k16);
                    a0 = mfma16x16x32(ah, bh, a0);
                    if constexpr (!FEAT) {
                        const bf16x8_t al = row_operand(sm.ql, QS, 16 * qt + c, 32 * s, g, 16);
                        const bf16x8_t bl = row_operand(sm.kl, KS, 16 * kt + c, 2 * k16 * s, g, k16);
                        a1 = mfma16x16x32(ah, bl, a1);
                        a2 = mfma16x16x32(al, bh, a2);
                    }
                }
                f32x4_t acc = a0 + (a1 + a2);
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
                        float rsum = acc[i];
                        rsum += __shfl_xor(rsum, 1, 64);
                        rsum += __shfl_xor(rsum, 2, 64);
                        rsum += __shfl_xor(rsum, 4, 64);
                        rsum += __shfl_xor(rsum, 8, 64);
                        if (c == 0) sm.denp[kt * TB + 16 * qt + 4 * g + i] = rsum;
                    }
                }
            }
        }
        __syncthreads();
        // fused gate: the previous block's sums were published at the top of
        // this block; start reading them now, use them after the products
        uint64_t xw[4];
        if constexpr (FUSE) {
            if (ti > 0 && wave == 0) gather_issue<TB>(ga, H, (uint32_t)ti, lane, xw);
        }

        // Matrix-core sections run at a raised wave priority (s_setprio 1):
        // with two workgroups per CU, the SIMD then issues the MFMA stream
        // of one wave first and fills its gaps with the other wave's vector
        // work (measured: main pass -4.5%).
        __builtin_amdgcn_s_setprio(1);
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
                    if constexpr (!FEAT) Al[dvt] = tr_operand(sm.vl, KS, 32 * ks, c0, g, c);
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
                            if constexpr (!FEAT)
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
                split2_keep(S[2 * s][dvt][0], S[2 * s][dvt][1], ah.x, al.x);
                split2_keep(S[2 * s][dvt][2], S[2 * s][dvt][3], ah.y, al.y);
                split2_keep(S[2 * s + 1][dvt][0], S[2 * s + 1][dvt][1], ah.z, al.z);
                split2_keep(S[2 * s + 1][dvt][2], S[2 * s + 1][dvt][3], ah.w, al.w);
                Ah[dvt] = as_bf16x8(ah);
                Al[dvt] = as_bf16x8(al);
            }
#pragma unroll
            for (int qt = 0; qt < L::NQT; ++qt) {
                if (qt < nqt) {
                    const bf16x8_t Bh = row_operand(sm.qh, QS, 16 * qt + c, 32 * s, g, 16);
                    if constexpr (FEAT) {
#pragma unroll
                        for (int dvt = 0; dvt < 2; ++dvt) {
                            acc[dvt][qt] = mfma16x16x32(Ah[dvt], Bh, acc[dvt][qt]);
                            acc[dvt][qt] = mfma16x16x32(Al[dvt], Bh, acc[dvt][qt]);
                        }
                    } else {
                        const bf16x8_t Bl = row_operand(sm.ql, QS, 16 * qt + c, 32 * s, g, 16);
#pragma unroll
                        for (int dvt = 0; dvt < 2; ++dvt) {
                            acc[dvt][qt] = mfma16x16x32(Ah[dvt], Bh, acc[dvt][qt]);
                            acc[dvt][qt] = mfma16x16x32(Ah[dvt], Bl, acc[dvt][qt]);
                            acc[dvt][qt] = mfma16x16x32(Al[dvt], Bh, acc[dvt][qt]);
                        }
                    }
                }
            }
        }
        __builtin_amdgcn_s_setprio(0);
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
        if constexpr (FUSE) {
            // the previous block: every head published its sums at the top
            // of this block
            if (ti > 0 && wave == 0) gather_finish<TB>(sm, ga, H, (uint32_t)ti, lane, xw);
        }
        __syncthreads();  // every wave's reads of this block's Q tile are done

        // ---- last phase: output, next block's Q tile, S += phi(K)^T phi(V) ----
        // (no branches on the data, so the vector work can interleave with
        // the state update's matrix-core work)
        OutT* yb = y + ((size_t)tt0 * H + h) * D;
        if constexpr (!FUSE) {
            const __amdgpu_buffer_rsrc_t ors = rows_rsrc(yb, rs * sizeof(OutT), D * sizeof(OutT), nvalid);
#pragma unroll
            for (int qt = 0; qt < L::NQT; ++qt) {
                if (qt < nqt) {
                    const uint32_t row = 16 * qt + c;
#pragma unroll
                    for (int dvt = 0; dvt < 2; ++dvt)
                        store4_buf<OutT>(ors, row * rs + 32 * wave + 16 * dvt + 4 * g, acc[dvt][qt]);
                }
            }
        }
        // the state update first: its LDS reads then precede the writes
        // below, which the compiler cannot prove disjoint from them
        __builtin_amdgcn_s_setprio(1);
        state_update<L::NKS, FEAT>(S, sm.kh, sm.kl, sm.vh, sm.vl, nks, wave, g, c);
        __builtin_amdgcn_s_setprio(0);
        if constexpr (FUSE) {
            // (for the first block nprev = 0: every store is dropped)
            gate_block<TB, OutT>(sm, rows_rsrc(ob, rs * sizeof(OutT), D * sizeof(OutT), nprev), xr,
                                 inv_f, ga.eps, rs, wave, g, c);
            stash_block<TB>(sm, acc, xr, rows_rsrc(xb, rs * 2u, D * 2u, nvalid), rs, wave, g, c);
            ob = yb;
            nprev = nvalid;
            xb += (size_t)TB * rs;
        }
        // rq holds block ti+1 (stale past the last block: staged, never read)
        stage_q<NORM, L::NJ, SmemMain<TB>, FEAT>(sm, rq, tid);
    }
    if constexpr (FUSE) {
        __syncthreads();
        publish_ssq<TB>(sm, ga, H, h, (uint32_t)ntiles);
        if (wave == 0) {
            uint64_t w[4];
            gather_issue<TB>(ga, H, (uint32_t)ntiles, lane, w);
            gather_finish<TB>(sm, ga, H, (uint32_t)ntiles, lane, w);
        }
        __syncthreads();
        gate_block<TB, OutT>(sm, rows_rsrc(ob, rs * sizeof(OutT), D * sizeof(OutT), nprev), xr, inv_f,
                             ga.eps, rs, wave, g, c);
    }

    if (it.last && it.row >= 0) {
        if (state_out) {
            float* dst = state_out + ((size_t)it.row * H + h) * D * D;
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
            if (tid < D) z_out[((size_t)it.row * H + h) * D + tid] = sm.z[tid];
        }
    }
}

// Unfused main pass: one workgroup per (chunk = blockIdx.x, head = blockIdx.y).
template <bool NORM, typename OutT, int TB, bool FEAT = false>
__global__ __launch_bounds__(NT, Tile<TB>::WG_PER_CU) void k_prefill_main(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    ItemMap map, int H, const float* __restrict__ prefix, int64_t prefix_stride,
    const float* __restrict__ state_in, const float* __restrict__ z_in, OutT* __restrict__ y,
    float* state_out, float* z_out, int k16) {
    __shared__ SmemMain<TB> sm;
    Item it;
    if (!decode_item(map, blockIdx.x, it)) return;
    GateArgs<uint16_t> ga{};
    process_item<NORM, false, OutT, uint16_t, TB, FEAT>(sm, q, k, v, it, blockIdx.x, H, blockIdx.y,
                                                   prefix, prefix_stride, state_in, z_in, y,
                                                   state_out, z_out, k16, ga);
}

// Fused main pass + gate, one workgroup per (chunk = blockIdx.x / H, head =
// blockIdx.x % H).  Launched cooperatively: every workgroup is resident, so
// the H heads of a chunk -- a team -- run together and their per-token sums
// of y^2 meet in the exchange buffer.  Every wait is bounded.
template <bool NORM, typename OutT, int TB, bool FEAT = false>
__global__ __launch_bounds__(NT, Tile<TB>::WG_PER_CU) void k_prefill_fused(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    ItemMap map, int H, const float* __restrict__ prefix, int64_t prefix_stride,
    const float* __restrict__ state_in, const float* __restrict__ z_in, OutT* __restrict__ out,
    float* state_out, float* z_out, int k16, const uint16_t* __restrict__ x,
    const float* __restrict__ w, float eps, uint64_t* xbuf, int spin_limit, uint32_t* status) {
    __shared__ SmemMain<TB> sm;
    const int item = blockIdx.x / H, h = blockIdx.x - item * H;
    Item it;
    if (!decode_item(map, item, it)) return;  // the whole team returns together
    GateArgs<uint16_t> ga{x, w, eps, xbuf, item, spin_limit, status};
    process_item<NORM, true, OutT, uint16_t, TB, FEAT>(sm, q, k, v, it, item, H, h, prefix,
                                                  prefix_stride, state_in, z_in, out, state_out,
                                                  z_out, k16, ga);
}

}  // namespace mf
}  // namespace la
