// proj_api.hip -- the C ABI of the layer's input and output projections
// (include/la_proj.h): host-side validation and the launch of the GEMM kernel
// (proj_kernels.h).
//
// Every argument check runs before the first HIP call, so a rejected call has
// no side effects.  The call allocates nothing.
#include "la_proj.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "proj_kernels.h"

using namespace la;

namespace {

inline bool dtype_arg_ok(const la_dtype_t& t, int& v) {
    static_assert(sizeof(la_dtype_t) == sizeof(int), "C enum size");
    std::memcpy(&v, &t, sizeof v);
    return v == LA_DTYPE_F32 || v == LA_DTYPE_BF16;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

inline bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || !na || !nb) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// Output tiles of 256 x 256 per call at most (the kernel indexes tiles and the
// grid in 32-bit integers).
constexpr int64_t kMaxTiles = (int64_t)1 << 28;

// Tile counts, the XCD-aware grid, and the launch (with the optional timing
// events around it).
la_status_t launch(pj::Args& a, int nblk, int odt, const la_proj_options_t& o, void* hip_stream) {
    const int64_t tm = ((int64_t)a.M + pj::BM - 1) / pj::BM, tn = (int64_t)nblk * a.F / pj::BN;
    const int64_t tiles = tm * tn;
    if (tiles > kMaxTiles) return LA_ERR_UNSUPPORTED;  // before any HIP call
    a.tiles_m = (int)tm;
    a.tiles_n = (int)tn;
    a.per_xcd = (int)((tiles + 7) / 8);
    hipStream_t st = (hipStream_t)hip_stream;
    hipEvent_t* ev = (hipEvent_t*)o.timing_events;
    if (ev && o.n_timing > 0) (void)hipEventRecord(ev[0], st);
    if (odt == LA_DTYPE_BF16)
        pj::k_proj<uint16_t><<<dim3((unsigned)(8 * a.per_xcd)), dim3(pj::NT), 0, st>>>(a);
    else
        pj::k_proj<float><<<dim3((unsigned)(8 * a.per_xcd)), dim3(pj::NT), 0, st>>>(a);
    if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
    if (ev && o.n_timing > 0) (void)hipEventRecord(ev[1], st);
    return LA_OK;
}

}  // namespace

extern "C" {

la_proj_options_t la_proj_default_options(void) {
    la_proj_options_t o;
    o.featurize = 1;
    o.timing_events = nullptr;
    o.n_timing = 0;
    return o;
}

la_status_t la_qkvx_projection(const void* hidden, const void* weight, void* q, void* k, void* v,
                               void* x_gate, int32_t T, int32_t K, int32_t F,
                               la_dtype_t out_dtype, const la_proj_options_t* opt,
                               void* hip_stream) {
    int odt = 0;
    if (!dtype_arg_ok(out_dtype, odt)) return LA_ERR_INVALID_ARGUMENT;
    const la_proj_options_t def = la_proj_default_options();
    const la_proj_options_t& o = opt ? *opt : def;
    if (o.featurize != 0 && o.featurize != 1) return LA_ERR_INVALID_ARGUMENT;
    if (o.n_timing < 0 || (o.n_timing > 0 && !o.timing_events)) return LA_ERR_INVALID_ARGUMENT;
    if (T < 0 || K < 1 || F < 1 || K > (1 << 20) || F > (1 << 20)) return LA_ERR_INVALID_ARGUMENT;
    if (K % pj::BK != 0 || F % pj::BN != 0) return LA_ERR_UNSUPPORTED;
    if (T == 0) return LA_OK;
    if (!hidden || !weight || !q || !k || !v) return LA_ERR_INVALID_ARGUMENT;
    const int nblk = x_gate ? 4 : 3;
    void* outs[4] = {q, k, v, x_gate};
    if (!aligned16(hidden) || !aligned16(weight)) return LA_ERR_INVALID_ARGUMENT;
    for (int i = 0; i < nblk; ++i)
        if (!aligned16(outs[i])) return LA_ERR_INVALID_ARGUMENT;
    const size_t osz = odt == LA_DTYPE_BF16 ? 2 : 4;
    const size_t in_bytes = (size_t)T * K * 2, w_bytes = (size_t)nblk * F * K * 2;
    const size_t out_bytes = (size_t)T * F * osz;
    for (int i = 0; i < nblk; ++i) {
        if (overlap(outs[i], out_bytes, hidden, in_bytes) || overlap(outs[i], out_bytes, weight, w_bytes))
            return LA_ERR_INVALID_ARGUMENT;
        for (int j = 0; j < i; ++j)
            if (overlap(outs[i], out_bytes, outs[j], out_bytes)) return LA_ERR_INVALID_ARGUMENT;
    }

    pj::Args a{};
    a.x = (const uint16_t*)hidden;
    a.w = (const uint16_t*)weight;
    for (int i = 0; i < 4; ++i) a.out[i] = outs[i];
    a.M = T;
    a.K = K;
    a.F = F;
    a.nsilu = o.featurize ? 3 : 0;
    return launch(a, nblk, odt, o, hip_stream);
}

la_status_t la_out_projection(const void* y, const void* weight, void* out, int32_t T, int32_t K,
                              int32_t N, la_dtype_t out_dtype, const la_proj_options_t* opt,
                              void* hip_stream) {
    int odt = 0;
    if (!dtype_arg_ok(out_dtype, odt)) return LA_ERR_INVALID_ARGUMENT;
    const la_proj_options_t def = la_proj_default_options();
    const la_proj_options_t& o = opt ? *opt : def;
    if (o.n_timing < 0 || (o.n_timing > 0 && !o.timing_events)) return LA_ERR_INVALID_ARGUMENT;
    if (T < 0 || K < 1 || N < 1 || K > (1 << 20) || N > (1 << 20)) return LA_ERR_INVALID_ARGUMENT;
    if (K % pj::BK != 0 || N % pj::BN != 0) return LA_ERR_UNSUPPORTED;
    if (T == 0) return LA_OK;
    if (!y || !weight || !out) return LA_ERR_INVALID_ARGUMENT;
    if (!aligned16(y) || !aligned16(weight) || !aligned16(out)) return LA_ERR_INVALID_ARGUMENT;
    const size_t osz = odt == LA_DTYPE_BF16 ? 2 : 4;
    if (overlap(out, (size_t)T * N * osz, y, (size_t)T * K * 2) ||
        overlap(out, (size_t)T * N * osz, weight, (size_t)N * K * 2))
        return LA_ERR_INVALID_ARGUMENT;

    pj::Args a{};
    a.x = (const uint16_t*)y;
    a.w = (const uint16_t*)weight;
    a.out[0] = out;
    a.M = T;
    a.K = K;
    a.F = N;  // one output block of N features
    a.nsilu = 0;
    return launch(a, 1, odt, o, hip_stream);
}

}  // extern "C"
