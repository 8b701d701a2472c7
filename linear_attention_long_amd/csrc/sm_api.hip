// sm_api.hip -- C ABI of the softmax attention layer (include/la_softmax.h):
// host-side validation, workspace layout and kernel launches.
//
// Every argument check runs on the host before the first HIP call, so a
// rejected call has no side effects.  The library allocates nothing.
#include "la_softmax.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "sm_kernels.h"

using namespace la;

namespace {

// Whether a dtype argument holds one of its declared values, read from its
// bytes: a C caller may pass any integer, and loading an out-of-range value
// through the enum type is undefined in C++.
inline bool dtype_arg_ok(const la_dtype_t& t) {
    static_assert(sizeof(la_dtype_t) == sizeof(int), "C enum size");
    int v;
    std::memcpy(&v, &t, sizeof v);
    return v == LA_DTYPE_F32 || v == LA_DTYPE_BF16;
}

#ifndef LA_SM_WAVES
#define LA_SM_WAVES 8
#endif
#ifndef LA_SM_WAVES_SPLIT
#define LA_SM_WAVES_SPLIT 8
#endif
// Waves per attention workgroup (32 queries each): single-operand mode
// LA_SM_WAVES, split mode LA_SM_WAVES_SPLIT; one workgroup per CU either way,
// two waves per SIMD with 8.
constexpr int kWavesPlain = LA_SM_WAVES;
constexpr int kWavesSplit = LA_SM_WAVES_SPLIT;
// fp16 operands: q, k and v are rounded to fp16 times this power of two
constexpr float kF16Pre = 0.015625f;  // 2^-6
inline int tile_queries(bool split) { return 32 * (split ? kWavesSplit : kWavesPlain); }

struct SmOpts {
    int rot;
    bool split;    // split operands (precision 1)
    bool f16;      // fp16 operands (precision 2)
    double base;
    float scale;
    hipEvent_t* events;
    int n_events;
};

struct SmLayout {
    int bq;           // queries per tile
    int ntmax;        // query tiles of the longest sequence
    int64_t emax;     // bound of the (sequence, tile) pairs
    bool planned;     // num_seqs > 1: the plan kernel orders the tiles
    size_t off_qr, off_kr, off_qrl, off_krl, off_vr, off_count, off_table, off_hist, off_off, off_cursor,
        off_tcu, total;
};

inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }
inline bool is_aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || !na || !nb) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

la_status_t sm_parse(const la_softmax_options_t* opt, int d, SmOpts& o) {
    const la_softmax_options_t def = la_softmax_default_options();
    const la_softmax_options_t& x = opt ? *opt : def;
    o.rot = x.rotary_dim == -1 ? d / 2 : x.rotary_dim;
    if (o.rot < 0 || o.rot > d || o.rot % 2) return LA_ERR_INVALID_ARGUMENT;
    if (o.rot % 16) return LA_ERR_UNSUPPORTED;
    o.base = x.rope_base;
    if (o.rot > 0 && !(std::isfinite(o.base) && o.base > 0.0)) return LA_ERR_INVALID_ARGUMENT;
    if (x.scale == 0.f) {
        o.scale = 1.0f / std::sqrt((float)d);
    } else {
        if (!(std::isfinite(x.scale) && x.scale > 0.f)) return LA_ERR_INVALID_ARGUMENT;
        o.scale = x.scale;
    }
    if (x.n_timing < 0 || (x.n_timing > 0 && !x.timing_events)) return LA_ERR_INVALID_ARGUMENT;
    o.events = (hipEvent_t*)x.timing_events;
    o.n_events = x.timing_events ? x.n_timing : 0;
    if (x.precision < 0 || x.precision > 2) return LA_ERR_INVALID_ARGUMENT;
    o.split = x.precision == 1;
    o.f16 = x.precision == 2;
    return LA_OK;
}

la_status_t sm_check(int32_t num_seqs, int32_t total_T, int32_t max_seqlen, int32_t H,
                     int32_t H_kv, int32_t d, la_dtype_t in_dtype, la_dtype_t out_dtype) {
    if (num_seqs < 1 || total_T < 0 || max_seqlen < 0 || max_seqlen > total_T)
        return LA_ERR_INVALID_ARGUMENT;
    if (H < 1 || H_kv < 1 || H % H_kv != 0 || d < 1) return LA_ERR_INVALID_ARGUMENT;
    if ((in_dtype != LA_DTYPE_F32 && in_dtype != LA_DTYPE_BF16) ||
        (out_dtype != LA_DTYPE_F32 && out_dtype != LA_DTYPE_BF16))
        return LA_ERR_INVALID_ARGUMENT;
    if (total_T > 0 && max_seqlen < 1) return LA_ERR_INVALID_ARGUMENT;
    if (d != sm::D || in_dtype != LA_DTYPE_BF16) return LA_ERR_UNSUPPORTED;
    if ((int64_t)H * d > (1 << 20)) return LA_ERR_UNSUPPORTED;
    return LA_OK;
}

la_status_t sm_layout(int32_t num_seqs, int32_t total_T, int32_t max_seqlen, int32_t H,
                      int32_t H_kv, bool split, bool f16, SmLayout& p) {
    const int BQ = tile_queries(split);
    p.bq = BQ;
    p.ntmax = (max_seqlen + BQ - 1) / BQ;
    p.planned = num_seqs > 1;
    const int64_t bound = ((int64_t)total_T + (int64_t)num_seqs * (BQ - 1)) / BQ;
    const int64_t dense = (int64_t)num_seqs * p.ntmax;
    p.emax = p.planned ? (dense < bound ? dense : bound) : p.ntmax;
    if (p.emax * H > INT32_MAX) return LA_ERR_UNSUPPORTED;
    size_t o = 0;
    p.off_qr = o;
    o = a256(o + (size_t)total_T * H * sm::D * 2);
    p.off_kr = o;
    o = a256(o + (size_t)total_T * H_kv * sm::D * 2);
    p.off_qrl = p.off_krl = p.off_vr = o;
    if (split) {  // bf16 remainders of the rotated q and k (precision 1)
        p.off_qrl = o;
        o = a256(o + (size_t)total_T * H * sm::D * 2);
        p.off_krl = o;
        o = a256(o + (size_t)total_T * H_kv * sm::D * 2);
    }
    if (f16) {  // v as fp16 (precision 2)
        p.off_vr = o;
        o = a256(o + (size_t)total_T * H_kv * sm::D * 2);
    }
    p.off_count = p.off_table = p.off_hist = p.off_off = p.off_cursor = p.off_tcu = o;
    if (p.planned) {
        p.off_count = o;
        o = a256(o + 4);
        p.off_table = o;
        o = a256(o + (size_t)p.emax * 8);
        p.off_hist = o;
        o = a256(o + (size_t)(p.ntmax + 1) * 4);
        p.off_off = o;
        o = a256(o + (size_t)p.ntmax * 4);
        p.off_cursor = o;
        o = a256(o + (size_t)p.ntmax * 4);
        p.off_tcu = o;
        o = a256(o + (size_t)(num_seqs + 1) * 4);
    }
    p.total = total_T > 0 ? o : 0;
    return LA_OK;
}

struct SmTimer {
    hipEvent_t* ev;
    int n;
    int i = 0;
    hipStream_t st;
    void before() {
        if (ev && i < n) (void)hipEventRecord(ev[2 * i], st);
    }
    void after() {
        if (ev && i < n) (void)hipEventRecord(ev[2 * i + 1], st);
        ++i;
    }
};

}  // namespace

extern "C" {

la_softmax_options_t la_softmax_default_options(void) {
    la_softmax_options_t o;
    o.rotary_dim = -1;
    o.rope_base = 10000.0;
    o.scale = 0.f;
    o.timing_events = nullptr;
    o.n_timing = 0;
    o.precision = 1;
    return o;
}

size_t la_softmax_workspace_bytes(int32_t num_seqs, int32_t total_T, int32_t max_seqlen,
                                  int32_t H, int32_t H_kv, int32_t d, la_dtype_t in_dtype,
                                  la_dtype_t out_dtype, const la_softmax_options_t* opt) {
    if (!dtype_arg_ok(in_dtype) || !dtype_arg_ok(out_dtype)) return (size_t)-1;
    if (sm_check(num_seqs, total_T, max_seqlen, H, H_kv, d, in_dtype, out_dtype) != LA_OK)
        return (size_t)-1;
    SmOpts o;
    if (sm_parse(opt, d, o) != LA_OK) return (size_t)-1;
    SmLayout p;
    if (sm_layout(num_seqs, total_T, max_seqlen, H, H_kv, o.split, o.f16, p) != LA_OK) return (size_t)-1;
    return p.total;
}

la_status_t la_softmax_attention_varlen(const void* q, const void* k, const void* v,
                                        const int32_t* cu_seqlens, int32_t num_seqs,
                                        int32_t total_T, int32_t max_seqlen, int32_t H,
                                        int32_t H_kv, int32_t d, la_dtype_t in_dtype,
                                        la_dtype_t out_dtype, void* out, float* lse,
                                        const la_softmax_options_t* opt, void* workspace,
                                        size_t workspace_bytes, void* hip_stream) {
    if (!dtype_arg_ok(in_dtype) || !dtype_arg_ok(out_dtype)) return LA_ERR_INVALID_ARGUMENT;
    la_status_t st = sm_check(num_seqs, total_T, max_seqlen, H, H_kv, d, in_dtype, out_dtype);
    if (st != LA_OK) return st;
    SmOpts o;
    if ((st = sm_parse(opt, d, o)) != LA_OK) return st;
    if (total_T == 0) return LA_OK;  // nothing to read or write
    if (!q || !k || !v || !cu_seqlens || !out) return LA_ERR_INVALID_ARGUMENT;
    if (!is_aligned(q, 16) || !is_aligned(k, 16) || !is_aligned(v, 16) || !is_aligned(out, 16) ||
        !is_aligned(cu_seqlens, 4) || (lse && !is_aligned(lse, 4)))
        return LA_ERR_INVALID_ARGUMENT;
    SmLayout p;
    if ((st = sm_layout(num_seqs, total_T, max_seqlen, H, H_kv, o.split, o.f16, p)) != LA_OK) return st;
    const size_t nq = (size_t)total_T * H * d * 2, nkv = (size_t)total_T * H_kv * d * 2;
    const size_t nout = (size_t)total_T * H * d * (out_dtype == LA_DTYPE_BF16 ? 2 : 4);
    const size_t nlse = lse ? (size_t)total_T * H * 4 : 0;
    const size_t ncu = (size_t)(num_seqs + 1) * 4;
    if (overlaps(out, nout, q, nq) || overlaps(out, nout, k, nkv) || overlaps(out, nout, v, nkv) ||
        overlaps(out, nout, cu_seqlens, ncu) || overlaps(out, nout, lse, nlse) ||
        overlaps(out, nout, workspace, p.total))
        return LA_ERR_INVALID_ARGUMENT;
    if (overlaps(lse, nlse, q, nq) || overlaps(lse, nlse, k, nkv) || overlaps(lse, nlse, v, nkv) ||
        overlaps(lse, nlse, cu_seqlens, ncu) || overlaps(lse, nlse, workspace, p.total))
        return LA_ERR_INVALID_ARGUMENT;
    if (overlaps(workspace, p.total, q, nq) || overlaps(workspace, p.total, k, nkv) ||
        overlaps(workspace, p.total, v, nkv) || overlaps(workspace, p.total, cu_seqlens, ncu))
        return LA_ERR_INVALID_ARGUMENT;
    if (p.total > 0) {
        if (!workspace || !is_aligned(workspace, 256)) return LA_ERR_INVALID_ARGUMENT;
        if (workspace_bytes < p.total) return LA_ERR_WORKSPACE_TOO_SMALL;
    }

    hipStream_t stream = (hipStream_t)hip_stream;
    SmTimer tm{o.events, o.n_events, 0, stream};
    char* ws = (char*)workspace;
    uint16_t* qr = (uint16_t*)(ws + p.off_qr);
    uint16_t* kr = (uint16_t*)(ws + p.off_kr);
    uint16_t* qrl = o.split ? (uint16_t*)(ws + p.off_qrl) : nullptr;
    uint16_t* krl = o.split ? (uint16_t*)(ws + p.off_krl) : nullptr;
    uint16_t* vr = o.f16 ? (uint16_t*)(ws + p.off_vr) : nullptr;
    const int2* table = nullptr;
    const int32_t* count = nullptr;
    if (p.planned) {
        tm.before();
        sm::k_sm_plan<<<1, 1024, 0, stream>>>(cu_seqlens, num_seqs, p.bq, p.ntmax,
                                               (int32_t*)(ws + p.off_hist),
                                               (int32_t*)(ws + p.off_off),
                                               (int32_t*)(ws + p.off_cursor),
                                               (int32_t*)(ws + p.off_tcu),
                                               (int2*)(ws + p.off_table),
                                               (int32_t*)(ws + p.off_count));
        tm.after();
        table = (const int2*)(ws + p.off_table);
        count = (const int32_t*)(ws + p.off_count);
    }
    {
        const int64_t want = ((int64_t)total_T + 15) / 16;
        const int grid = (int)(want < 16384 ? want : 16384);
        // scores in log2 units: q carries scale * log2(e), except with split
        // or fp16 operands, where the attention kernel scales the fp32 scores
        // (split: q then stays exact outside the rotated dimensions).  fp16
        // q, k and v are taken times 2^-6 (exact), which moves fp16's normal
        // range to elements in [2^-8, 2^22); the attention kernel multiplies
        // the scores back by 2^12 and the output by 2^6.
        const float qscale = o.f16 ? kF16Pre : o.split ? 1.0f : o.scale * 1.4426950408889634f;
        const float kscale = o.f16 ? kF16Pre : 1.0f;
        tm.before();
        sm::k_sm_rope<<<grid, 256, 0, stream>>>((const uint16_t*)q, (const uint16_t*)k, cu_seqlens,
                                                num_seqs, total_T, H, H_kv, o.rot,
                                                o.rot > 0 ? std::log2(o.base) : 0.0, qscale, kscale,
                                                qr, kr, qrl, krl, o.f16 ? 1 : 0,
                                                (const uint16_t*)v, vr, kF16Pre);
        tm.after();
    }
    const unsigned grid = (unsigned)(p.emax * H);
    tm.before();
    if (grid > 0) {
        const float qs = o.scale * 1.4426950408889634f * (o.f16 ? 1.0f / (kF16Pre * kF16Pre) : 1.0f);
        const float ovs = o.f16 ? 1.0f / kF16Pre : 1.0f;
        const uint16_t* vin = o.f16 ? vr : (const uint16_t*)v;
        const int nrk = (o.rot + 31) / 32;  // 32-dimension steps holding rotated dimensions
#define SM_ATTN(OT, SP, W, NRK, F16)                                                                \
    sm::k_sm_attn<OT, SP, W, NRK, F16><<<grid, 64 * W, 0, stream>>>(qr, kr, qrl, krl, vin,           \
                                                               cu_seqlens, table, count, H, H_kv,   \
                                                               (OT*)out, lse, qs, ovs)
#define SM_ATTN_SPLIT(OT)                                           \
    switch (nrk) {                                                  \
        case 0: SM_ATTN(OT, true, kWavesSplit, 0, false); break;    \
        case 1: SM_ATTN(OT, true, kWavesSplit, 1, false); break;    \
        case 2: SM_ATTN(OT, true, kWavesSplit, 2, false); break;    \
        case 3: SM_ATTN(OT, true, kWavesSplit, 3, false); break;    \
        default: SM_ATTN(OT, true, kWavesSplit, 4, false); break;   \
    }
        if (out_dtype == LA_DTYPE_BF16) {
            if (o.split) { SM_ATTN_SPLIT(uint16_t) }
            else if (o.f16) SM_ATTN(uint16_t, false, kWavesPlain, 4, true);
            else SM_ATTN(uint16_t, false, kWavesPlain, 4, false);
        } else {
            if (o.split) { SM_ATTN_SPLIT(float) }
            else if (o.f16) SM_ATTN(float, false, kWavesPlain, 4, true);
            else SM_ATTN(float, false, kWavesPlain, 4, false);
        }
#undef SM_ATTN_SPLIT
#undef SM_ATTN
    }
    tm.after();
    return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

}  // extern "C"
