// la_api.hip -- the C ABI of liblinattn (declared in include/la.h): host-side
// validation, planning of chunks and workspace, and kernel launches.
//
// Every argument check runs on the host before the first HIP call, so a
// rejected call has no side effects.  The library allocates nothing.
#include "la.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "la_kernels_aux.h"
#include "la_kernels_mfma.h"
#include "la_kernels_valu.h"

using namespace la;

// ---- scratch of the entry point that allocates nothing (la_prefill_noalloc) ----
// One array per GPU, for the life of the process.  In host code `scratch`
// names a host-side stand-in, not device memory: its device address comes
// from hipGetSymbolAddress, once per device, and only that address is ever
// passed to kernels.
static __device__ __align__(256) unsigned char scratch[LA_NOALLOC_SCRATCH_BYTES];

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

constexpr int kMfmaDefaultBlock = 32;   // bf16 d=128: two workgroups per CU
constexpr int kValuDefaultBlock = 64;
constexpr int kMinAutoChunk = 512;
constexpr int kMaxAutoChunk = 16384;
constexpr int64_t kTargetItems = 2048;  // (chunk, head) workgroups aimed for: ~4 per CU slot
// Fused plans with chunks of at least this many tokens run the chunk-state
// pass on half chunks, with the one-buffer kernel at four workgroups per CU
// (the scan adds the two halves): the fused pass sizes its chunks for one
// resident round of two workgroups per CU, the state pass runs better with
// more, smaller workgroups.
constexpr int kSubChunkMin = 8192;
constexpr int kSpinLimit = 1 << 22;     // bounded waits of the fused gate (~seconds)
constexpr size_t kStatusBytes = 256;    // the call's device status word, padded
#ifndef LA_DECODE_SPLIT
#define LA_DECODE_SPLIT 4
#endif
constexpr int kDecodeSplit = LA_DECODE_SPLIT;  // decode workgroups per (sequence, head), plain mode
constexpr int64_t kStreamStateBytes = (int64_t)64 << 20;  // decode: stream states at least this large

// Workgroups of `kernel` (256 threads) the current device keeps resident at
// once, or 0 when cooperative launch is unavailable.
int64_t resident_capacity(const void* kernel) {
    int dev = 0, ncu = 0, coop = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess || !coop)
        return 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess) return 0;
    return (int64_t)per_cu * ncu;
}

struct Opts {
    int block;
    bool normalized;
    bool gated;
    int group;      // RMSNorm group width (features)
    float eps;
    int chunk;      // requested chunk tokens (0 = auto)
    hipEvent_t* events;
    int n_events;
    const int32_t* slots;  // state row per sequence (device), or nullptr
    int rows;              // rows of the state arrays when slots is given
    bool feat;             // q, k, v are feature vectors already (no SiLU inside)
    int spin;              // retries per bounded wait of the fused gate (< 0: none)
    int state_access;      // decode: 0 auto, 1 streaming (non-temporal), 2 cache-resident
};

// Records the caller's timing events around each launched kernel.
struct Timer {
    hipEvent_t* ev;
    int n;
    int i = 0;
    hipStream_t st;
    Timer(const Opts& o, hipStream_t s) : ev(o.events), n(o.n_events), st(s) {}
    void before() {
        if (ev && i < n) (void)hipEventRecord(ev[2 * i], st);
    }
    void after() {
        if (ev && i < n) (void)hipEventRecord(ev[2 * i + 1], st);
        ++i;
    }
};

struct Plan {
    bool fuse_ok;      // gated bf16 d=128 block 32 with H <= 8: gate fused into the main pass
    int64_t xbuf_words;  // exchange buffer of the fused gate (64-bit words)
    size_t off_xbuf;     // fused: [status word (256 B) | exchange buffer], cleared together
    int block;         // resolved block size
    bool mfma;         // bf16, d = 128, block 32 or 64: matrix-core kernels
    bool chunked;      // some sequence spans more than one chunk
    bool varlen;
    int C;             // tokens per chunk
    int64_t items;     // grid size bound in chunks
    int64_t stride;    // floats per (item, head) in the state buffer
    bool cdev;         // varlen, fused: the chunk length is searched on the device (<= C)
    int c_lo;          // its lower bound
    int64_t teams;     // fused: resident (chunk, head) teams = items bound
    bool half;         // chunk-state pass on half chunks (equal lengths, fused, C >= kSubChunkMin)
    int cps2;          // its half chunks per sequence
    int64_t items2;    // and their count
    size_t off_chunk_off, off_buf, off_part, off_y, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
inline bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || !na || !nb) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}
inline size_t dtype_size(la_dtype_t t) { return t == LA_DTYPE_BF16 ? 2 : 4; }
inline bool dtype_ok(la_dtype_t t) { return t == LA_DTYPE_F32 || t == LA_DTYPE_BF16; }

la_status_t parse_options(const la_options_t* opt, int H, int d, Opts& o) {
    const la_options_t def = la_default_options();
    const la_options_t& x = opt ? *opt : def;
    o.block = x.block_size;
    if (o.block != 0 && o.block != 32 && o.block != 64 && o.block != 128 && o.block != 256)
        return LA_ERR_UNSUPPORTED;
    if (x.normalized != 0 && x.normalized != 1) return LA_ERR_INVALID_ARGUMENT;
    if (x.gated != 0 && x.gated != 1) return LA_ERR_INVALID_ARGUMENT;
    o.normalized = x.normalized == 1;
    o.gated = x.gated == 1;
    const int F = H * d;
    o.group = x.norm_group == 0 ? F : x.norm_group;
    if (o.group <= 0 || o.group % 64 != 0 || F % o.group != 0) return LA_ERR_INVALID_ARGUMENT;
    if (!(x.rms_eps >= 0.f) || !std::isfinite(x.rms_eps)) return LA_ERR_INVALID_ARGUMENT;
    o.eps = x.rms_eps;
    if (x.chunk_tokens < 0 || x.chunk_tokens % 64 != 0) return LA_ERR_INVALID_ARGUMENT;
    o.chunk = x.chunk_tokens;
    if (x.n_timing < 0 || (x.n_timing > 0 && !x.timing_events)) return LA_ERR_INVALID_ARGUMENT;
    o.events = (hipEvent_t*)x.timing_events;
    o.n_events = x.timing_events ? x.n_timing : 0;
    o.slots = x.state_slots;
    o.rows = x.state_slots ? x.state_rows : 0;
    if (x.state_slots && (x.state_rows < 1 || !aligned(x.state_slots, 4))) return LA_ERR_INVALID_ARGUMENT;
    if (x.featurized != 0 && x.featurized != 1) return LA_ERR_INVALID_ARGUMENT;
    o.feat = x.featurized == 1;
    if (x.wait_spin_limit < -1) return LA_ERR_INVALID_ARGUMENT;
    o.spin = x.wait_spin_limit == 0 ? kSpinLimit : x.wait_spin_limit;
    if (x.state_access < 0 || x.state_access > 2) return LA_ERR_INVALID_ARGUMENT;
    o.state_access = x.state_access;
    return LA_OK;
}

la_status_t check_shape(int32_t H, int32_t d, la_dtype_t in_dtype, la_dtype_t out_dtype) {
    if (H < 1 || d < 1) return LA_ERR_INVALID_ARGUMENT;
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return LA_ERR_INVALID_ARGUMENT;
    if (d != 64 && d != 128) return LA_ERR_UNSUPPORTED;
    if ((int64_t)H * d > (1 << 20)) return LA_ERR_UNSUPPORTED;
    return LA_OK;
}

int auto_chunk(int64_t total_T, int H, int max_seqlen, const Opts& o) {
    if (o.chunk) return o.chunk;
    int64_t C = (total_T * H + kTargetItems - 1) / kTargetItems;
    C = (C + 63) / 64 * 64;
    if (C < kMinAutoChunk) C = kMinAutoChunk;
    if (C > kMaxAutoChunk) C = kMaxAutoChunk;
    (void)max_seqlen;
    return (int)C;
}

int64_t items_for(bool varlen, int64_t num_seqs, int64_t total_T, int64_t max_seqlen, int64_t C) {
    return varlen ? total_T / C + num_seqs : num_seqs * ((max_seqlen + C - 1) / C);
}

// The fused main pass + gate for these options (32-token blocks).
const void* fused_kernel(bool norm, bool f32_out, bool feat) {
    if (feat)
        return norm ? (f32_out ? (const void*)mf::k_prefill_fused<true, float, 32, true>
                               : (const void*)mf::k_prefill_fused<true, uint16_t, 32, true>)
                    : (f32_out ? (const void*)mf::k_prefill_fused<false, float, 32, true>
                               : (const void*)mf::k_prefill_fused<false, uint16_t, 32, true>);
    return norm ? (f32_out ? (const void*)mf::k_prefill_fused<true, float, 32>
                           : (const void*)mf::k_prefill_fused<true, uint16_t, 32>)
                : (f32_out ? (const void*)mf::k_prefill_fused<false, float, 32>
                           : (const void*)mf::k_prefill_fused<false, uint16_t, 32>);
}

Plan make_plan(bool varlen, int64_t num_seqs, int64_t total_T, int64_t max_seqlen, int H, int d,
               la_dtype_t in_dtype, la_dtype_t out_dtype, const Opts& o, bool allow_half = true) {
    Plan p{};
    p.varlen = varlen;
    p.block = o.block;
    if (p.block == 0) p.block = (in_dtype == LA_DTYPE_BF16 && d == 128) ? kMfmaDefaultBlock : kValuDefaultBlock;
    p.mfma = in_dtype == LA_DTYPE_BF16 && d == 128 && (p.block == 32 || p.block == 64);
    p.stride = (int64_t)d * d + (o.normalized ? d : 0);
    // Fused gate: every (chunk, head) workgroup must be resident at once, so the
    // chunk length is chosen for (chunks x H) <= the device's capacity.
    p.fuse_ok = false;
    // (the fused gate normalises over all H*d features of a token)
    const bool fusable = o.gated && o.group == H * d && p.mfma && p.block == 32 &&
                         H <= mf::FUSE_HMAX && total_T > 0;
    const void* fk = fused_kernel(o.normalized, true, o.feat);
    const int64_t cap = fusable ? resident_capacity(fk) : 0;
    if (cap >= H) {
        const int64_t teams = cap / H;
        int64_t C;
        if (o.chunk) {
            C = o.chunk;
        } else if (varlen) {
            C = teams > num_seqs ? (total_T + (teams - num_seqs) - 1) / (teams - num_seqs) : 0;
        } else {
            const int64_t per_seq = teams / num_seqs;
            C = per_seq > 0 ? (max_seqlen + per_seq - 1) / per_seq : 0;
        }
        C = (C + 63) / 64 * 64;
        if (C > 0 && C < (int64_t)1 << 30) {
            if (!o.chunk && C < kMinAutoChunk) C = kMinAutoChunk;
            if (max_seqlen <= C) C = max_seqlen <= 64 ? 64 : (max_seqlen + 63) / 64 * 64;
            const int64_t items = items_for(varlen, num_seqs, total_T, max_seqlen, C);
            if (items <= teams) {
                p.fuse_ok = true;
                p.C = (int)C;
                p.teams = teams;
            }
        }
    }
    if (!p.fuse_ok) p.C = auto_chunk(total_T, H, (int)max_seqlen, o);
    p.chunked = max_seqlen > p.C;
    if (!p.chunked) {
        // one chunk per sequence: the chunk length only has to cover it
        int64_t c = (max_seqlen + 63) / 64 * 64;
        p.C = (int)(c < 64 ? 64 : c);
    }
    p.items = items_for(varlen, num_seqs, total_T, max_seqlen, p.C);
    p.half = allow_half && p.fuse_ok && !varlen && p.chunked && p.C >= kSubChunkMin;
    p.cps2 = p.half ? (int)((max_seqlen + p.C / 2 - 1) / (p.C / 2)) : 0;
    p.items2 = p.half ? (int64_t)num_seqs * p.cps2 : 0;
    // Fused varlen batches whose sequences span chunks: C above is sized for
    // the worst case of the lengths (every sequence ends in a short chunk);
    // the chunk planner searches, on the device, the smallest chunk length
    // (multiple of 64, at least kMinAutoChunk unless C is smaller) whose
    // chunk count still fits the resident teams.
    p.cdev = varlen && p.fuse_ok && p.chunked && !o.chunk;
    if (p.cdev) {
        int64_t lo = (total_T + p.teams - 1) / p.teams;
        lo = (lo + 63) / 64 * 64;
        if (lo < kMinAutoChunk) lo = kMinAutoChunk;
        p.c_lo = (int)(lo < p.C ? lo : p.C);
        p.items = p.teams;
    }
    p.xbuf_words = p.fuse_ok ? p.items * mf::NSLOT * H * 32 : 0;
    size_t off = 0;
    p.off_chunk_off = off;
    if (varlen) off += align256((size_t)(num_seqs + 2) * sizeof(int32_t));
    p.off_buf = off;
    if (p.chunked) off += align256((size_t)p.items * H * p.stride * sizeof(float));
    p.off_part = off;
    if (p.half) off += align256((size_t)p.items2 * H * p.stride * sizeof(float));
    p.off_y = off;
    if (o.gated && out_dtype != LA_DTYPE_F32 && !p.fuse_ok)
        off += align256((size_t)total_T * H * d * sizeof(float));
    p.off_xbuf = off;
    if (p.fuse_ok) off += kStatusBytes + align256((size_t)p.xbuf_words * sizeof(uint64_t));
    p.total = off;
    return p;
}

// Gate kernel choice: registers-resident groups of 256/512/1024/2048 features,
// else the general loop.
template <typename XT, typename OT>
void launch_gate(unsigned blocks, hipStream_t st, const float* y, const XT* x, const float* w,
                 OT* out, int64_t ntok, int F, int G, float eps) {
    switch (G) {
        case 256: k_gate4<XT, OT, 1><<<blocks, 256, 0, st>>>(y, x, w, out, ntok, F, G, eps); break;
        case 512: k_gate4<XT, OT, 2><<<blocks, 256, 0, st>>>(y, x, w, out, ntok, F, G, eps); break;
        case 1024: k_gate4<XT, OT, 4><<<blocks, 256, 0, st>>>(y, x, w, out, ntok, F, G, eps); break;
        case 2048: k_gate4<XT, OT, 8><<<blocks, 256, 0, st>>>(y, x, w, out, ntok, F, G, eps); break;
        default: k_gate<XT, OT><<<blocks, 256, 0, st>>>(y, x, w, out, ntok, F, G, eps); break;
    }
}

template <typename InT, typename OutT>
la_status_t launch_prefill_typed(const Plan& p, const Opts& o, const void* q, const void* k,
                                 const void* v, const void* x, const float* w,
                                 const int32_t* cu, int32_t nseq, int32_t T, int64_t total_T,
                                 const float* state_in, const float* z_in, void* out,
                                 float* state_out, float* z_out, int H, int d, char* ws,
                                 hipStream_t st) {
    Timer tm(o, st);
    ItemMap map{};
    map.nseq = nseq;
    map.C = p.C;
    map.slots = o.slots;
    map.rows = o.rows;
    if (p.varlen) {
        map.cu = cu;
        map.chunk_off = (int32_t*)(ws + p.off_chunk_off);
        tm.before();
        k_plan_chunks<<<1, 256, 0, st>>>(cu, nseq, p.C, (int32_t*)(ws + p.off_chunk_off),
                                         p.cdev ? 1 : 0, p.c_lo, (int32_t)p.teams);
        map.cdev = p.cdev ? 1 : 0;
        if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
        tm.after();
    } else {
        map.T = T;
        map.cps = (T + p.C - 1) / p.C;
    }
    if (total_T == 0 || (p.varlen && !p.chunked)) {
        // zero-length sequences keep their state; others are overwritten below
        if (state_out || z_out) {
            tm.before();
            k_fill_state<<<dim3((unsigned)((d * d + d + 255) / 256), (unsigned)((int64_t)nseq * H)), 256, 0, st>>>(
                state_in, z_in, state_out, o.normalized ? z_out : nullptr, map, H, d);
            if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
            tm.after();
        }
        if (total_T == 0) return LA_OK;
    }
    const bool need_yws = o.gated && !p.fuse_ok && !std::is_same<OutT, float>::value;
    float* ybuf_f = need_yws ? (float*)(ws + p.off_y) : nullptr;
    float* buf = p.chunked ? (float*)(ws + p.off_buf) : nullptr;
    const dim3 grid((unsigned)p.items, (unsigned)H);
    const bool norm = o.normalized;

    if (p.chunked) {
        tm.before();
        if (p.mfma) {
            if (p.half) {
                const auto ck1 = norm ? (o.feat ? mf::k_chunk_state1<true, true> : mf::k_chunk_state1<true, false>)
                                      : (o.feat ? mf::k_chunk_state1<false, true> : mf::k_chunk_state1<false, false>);
                ItemMap m2 = map;
                m2.C = p.C / 2;
                m2.cps = p.cps2;
                ck1<<<dim3((unsigned)p.items2, (unsigned)H), mf::NT, 0, st>>>(
                    (const uint16_t*)k, (const uint16_t*)v, m2, H, (float*)(ws + p.off_part), p.stride);
            } else {
                const auto ck = norm ? (o.feat ? mf::k_chunk_state<true, true> : mf::k_chunk_state<true, false>)
                                     : (o.feat ? mf::k_chunk_state<false, true> : mf::k_chunk_state<false, false>);
                ck<<<grid, mf::NT, 0, st>>>((const uint16_t*)k, (const uint16_t*)v, map, H, buf, p.stride);
            }
        } else if (d == 128) {
            if (norm) vk::k_valu_state<128, InT, true><<<grid, vk::NT, 0, st>>>((const InT*)k, (const InT*)v, map, H, buf, p.stride, o.feat ? 1 : 0);
            else vk::k_valu_state<128, InT, false><<<grid, vk::NT, 0, st>>>((const InT*)k, (const InT*)v, map, H, buf, p.stride, o.feat ? 1 : 0);
        } else {
            if (norm) vk::k_valu_state<64, InT, true><<<grid, vk::NT, 0, st>>>((const InT*)k, (const InT*)v, map, H, buf, p.stride, o.feat ? 1 : 0);
            else vk::k_valu_state<64, InT, false><<<grid, vk::NT, 0, st>>>((const InT*)k, (const InT*)v, map, H, buf, p.stride, o.feat ? 1 : 0);
        }
        if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
        tm.after();
        const int E = (int)p.stride;
        const int nblk = (E + 255) / 256;
        tm.before();
        k_chunk_scan<<<dim3((unsigned)nblk, (unsigned)H, (unsigned)nseq), 256, 0, st>>>(
            buf, p.stride, map, H, d, E, state_in, norm ? z_in : nullptr, state_out,
            norm ? z_out : nullptr, p.fuse_ok ? (uint64_t*)(ws + p.off_xbuf) : nullptr,
            p.fuse_ok ? p.xbuf_words + (int64_t)(kStatusBytes / 8) : 0,
            p.half ? (const float*)(ws + p.off_part) : nullptr, p.cps2);
        if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
        tm.after();
    }

    // main pass: Y in the output dtype, or fp32 (out itself when fp32) when gated
    // fused gate: one cooperative launch, every (chunk, head) workgroup resident
    if (p.fuse_ok) {
        const bool f32o = std::is_same<OutT, float>::value;
        const void* kern = fused_kernel(norm, f32o, o.feat);
        uint32_t* status = (uint32_t*)(ws + p.off_xbuf);
        uint64_t* xbuf = (uint64_t*)(ws + p.off_xbuf + kStatusBytes);
        const int64_t nw = p.xbuf_words + (int64_t)(kStatusBytes / 8);
        if (!p.chunked) {  // (a chunked call's scan cleared it)
            tm.before();
            k_zero_u64<<<(unsigned)((nw + 255) / 256), 256, 0, st>>>((uint64_t*)status, nw);
            if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
            tm.after();
        }
        const uint16_t* qb = (const uint16_t*)q;
        const uint16_t* kb = (const uint16_t*)k;
        const uint16_t* vb = (const uint16_t*)v;
        const uint16_t* xb = (const uint16_t*)x;
        int k16 = 16, spin = o.spin, Hh = H;
        float eps = o.eps;
        float* so = state_out;  // written after each sequence's last chunk
        float* zo = norm ? z_out : nullptr;
        const float* bufc = buf;
        int64_t stride = p.stride;
        OutT* outp = (OutT*)out;
        void* args[] = {(void*)&qb, (void*)&kb, (void*)&vb, (void*)&map, (void*)&Hh,
                        (void*)&bufc, (void*)&stride, (void*)&state_in, (void*)&z_in,
                        (void*)&outp, (void*)&so, (void*)&zo, (void*)&k16, (void*)&xb,
                        (void*)&w, (void*)&eps, (void*)&xbuf, (void*)&spin, (void*)&status};
        tm.before();
        const hipError_t e = hipLaunchCooperativeKernel(kern, dim3((unsigned)(p.items * H)),
                                                        dim3(mf::NT), args, 0, st);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return LA_ERR_HIP;
        }
        tm.after();
        return LA_OK;
    }

    void* ydst = o.gated ? (need_yws ? (void*)ybuf_f : out) : out;
    const bool y_is_f32 = o.gated || std::is_same<OutT, float>::value;
    tm.before();
    if (p.mfma) {
        const uint16_t* qb = (const uint16_t*)q;
        const uint16_t* kb = (const uint16_t*)k;
        const uint16_t* vb = (const uint16_t*)v;
        float* so = state_out;  // written after each sequence's last chunk
        float* zo = z_out;
#define LA_MF_MAIN(NN, YT, TBV) \
    mf::k_prefill_main<NN, YT, TBV><<<grid, mf::NT, 0, st>>>(qb, kb, vb, map, H, buf, p.stride, state_in, z_in, (YT*)ydst, so, NN ? zo : nullptr, 16)
#define LA_MF_MAIN_F(NN, YT) \
    mf::k_prefill_main<NN, YT, 32, true><<<grid, mf::NT, 0, st>>>(qb, kb, vb, map, H, buf, p.stride, state_in, z_in, (YT*)ydst, so, NN ? zo : nullptr, 16)
        if (o.feat) {  // (the checks admit block 32 only on this path)
            if (y_is_f32) { if (norm) LA_MF_MAIN_F(true, float); else LA_MF_MAIN_F(false, float); }
            else { if (norm) LA_MF_MAIN_F(true, uint16_t); else LA_MF_MAIN_F(false, uint16_t); }
        } else if (p.block == 32) {
            if (y_is_f32) { if (norm) LA_MF_MAIN(true, float, 32); else LA_MF_MAIN(false, float, 32); }
            else { if (norm) LA_MF_MAIN(true, uint16_t, 32); else LA_MF_MAIN(false, uint16_t, 32); }
        } else {
            if (y_is_f32) { if (norm) LA_MF_MAIN(true, float, 64); else LA_MF_MAIN(false, float, 64); }
            else { if (norm) LA_MF_MAIN(true, uint16_t, 64); else LA_MF_MAIN(false, uint16_t, 64); }
        }
#undef LA_MF_MAIN
#undef LA_MF_MAIN_F
    } else {
#define LA_VALU_MAIN(DD, YT, NN)                                                                \
    vk::k_valu_main<DD, InT, YT, NN><<<grid, vk::NT, 0, st>>>(                                  \
        (const InT*)q, (const InT*)k, (const InT*)v, map, H, p.block, buf, p.stride, state_in,  \
        z_in, (YT*)ydst, state_out, z_out, o.feat ? 1 : 0)
        if (d == 128) {
            if (y_is_f32) { if (norm) LA_VALU_MAIN(128, float, true); else LA_VALU_MAIN(128, float, false); }
            else { if (norm) LA_VALU_MAIN(128, uint16_t, true); else LA_VALU_MAIN(128, uint16_t, false); }
        } else {
            if (y_is_f32) { if (norm) LA_VALU_MAIN(64, float, true); else LA_VALU_MAIN(64, float, false); }
            else { if (norm) LA_VALU_MAIN(64, uint16_t, true); else LA_VALU_MAIN(64, uint16_t, false); }
        }
#undef LA_VALU_MAIN
    }
    if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
    tm.after();

    if (o.gated) {
        const int F = H * d;
        const int64_t units = total_T * (F / o.group);
        const unsigned blocks = (unsigned)((units + 3) / 4);
        const float* yf = need_yws ? ybuf_f : (const float*)out;
        tm.before();
        launch_gate<InT, OutT>(blocks, st, yf, (const InT*)x, w, (OutT*)out, total_T, F, o.group, o.eps);
        if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
        tm.after();
    }
    return LA_OK;
}

la_status_t launch_prefill(const Plan& p, const Opts& o, la_dtype_t in_dtype, la_dtype_t out_dtype,
                           const void* q, const void* k, const void* v, const void* x,
                           const float* w, const int32_t* cu, int32_t nseq, int32_t T,
                           int64_t total_T, const float* state_in, const float* z_in, void* out,
                           float* state_out, float* z_out, int H, int d, char* ws, hipStream_t st) {
    if (in_dtype == LA_DTYPE_BF16) {
        if (out_dtype == LA_DTYPE_BF16)
            return launch_prefill_typed<uint16_t, uint16_t>(p, o, q, k, v, x, w, cu, nseq, T, total_T, state_in, z_in, out, state_out, z_out, H, d, ws, st);
        return launch_prefill_typed<uint16_t, float>(p, o, q, k, v, x, w, cu, nseq, T, total_T, state_in, z_in, out, state_out, z_out, H, d, ws, st);
    }
    if (out_dtype == LA_DTYPE_BF16)
        return launch_prefill_typed<float, uint16_t>(p, o, q, k, v, x, w, cu, nseq, T, total_T, state_in, z_in, out, state_out, z_out, H, d, ws, st);
    return launch_prefill_typed<float, float>(p, o, q, k, v, x, w, cu, nseq, T, total_T, state_in, z_in, out, state_out, z_out, H, d, ws, st);
}

// Checks shared by both prefill entry points.
// Inputs given as features: every prefill configuration except the bf16
// d = 128 matrix-core pass with 64-token blocks (its kernels have no such
// variant).
bool feat_unsupported(const Opts& o, la_dtype_t in_dtype, int d) {
    return o.feat && in_dtype == LA_DTYPE_BF16 && d == 128 && o.block == 64;
}

la_status_t check_prefill_common(const void* q, const void* k, const void* v, const void* x_gate,
                                 const float* rms_weight, const float* state_in, const float* z_in,
                                 void* out, float* state_out, float* z_out, int64_t nseq,
                                 int64_t total_T, int H, int d, la_dtype_t in_dtype,
                                 la_dtype_t out_dtype, const Opts& o) {
    if (feat_unsupported(o, in_dtype, d)) return LA_ERR_UNSUPPORTED;
    if (!q || !k || !v || !out) return LA_ERR_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return LA_ERR_INVALID_ARGUMENT;
    if (o.gated && (!x_gate || !aligned(x_gate, 16))) return LA_ERR_INVALID_ARGUMENT;
    if (rms_weight && !aligned(rms_weight, 16)) return LA_ERR_INVALID_ARGUMENT;
    if (!o.normalized && (z_in || z_out)) return LA_ERR_INVALID_ARGUMENT;
    const void* st_ptrs[4] = {state_in, z_in, state_out, z_out};
    for (const void* sp : st_ptrs)
        if (sp && !aligned(sp, 16)) return LA_ERR_INVALID_ARGUMENT;
    const size_t in_bytes = (size_t)total_T * H * d * dtype_size(in_dtype);
    const size_t out_bytes = (size_t)total_T * H * d * dtype_size(out_dtype);
    const int64_t srows = o.slots ? o.rows : nseq;  // rows of the state arrays
    const size_t s_bytes = (size_t)srows * H * d * d * sizeof(float);
    const size_t z_bytes = (size_t)srows * H * d * sizeof(float);
    const void* ins[4] = {q, k, v, o.gated ? x_gate : nullptr};
    for (const void* ip : ins)
        if (overlap(out, out_bytes, ip, in_bytes)) return LA_ERR_INVALID_ARGUMENT;
    if (overlap(out, out_bytes, state_out, s_bytes) || overlap(out, out_bytes, state_in, s_bytes))
        return LA_ERR_INVALID_ARGUMENT;
    if (state_out && state_in && state_out != state_in && overlap(state_out, s_bytes, state_in, s_bytes))
        return LA_ERR_INVALID_ARGUMENT;
    if (z_out && z_in && z_out != z_in && overlap(z_out, z_bytes, z_in, z_bytes))
        return LA_ERR_INVALID_ARGUMENT;
    if (state_out && overlap(state_out, s_bytes, z_out, z_bytes)) return LA_ERR_INVALID_ARGUMENT;
    return LA_OK;
}

la_status_t check_workspace(const Plan& p, void* ws, size_t ws_bytes) {
    if (p.total == 0) return LA_OK;
    if (!ws || !aligned(ws, 256)) return LA_ERR_INVALID_ARGUMENT;
    if (ws_bytes < p.total) return LA_ERR_WORKSPACE_TOO_SMALL;
    return LA_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up on the first call on
// that device; nullptr on failure.
void* scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

la_options_t la_default_options(void) {
    la_options_t o;
    o.block_size = 0;
    o.normalized = 0;
    o.gated = 0;
    o.norm_group = 0;
    o.rms_eps = 1e-6f;
    o.chunk_tokens = 0;
    o.timing_events = nullptr;
    o.n_timing = 0;
    o.state_slots = nullptr;
    o.state_rows = 0;
    o.featurized = 0;
    o.wait_spin_limit = 0;
    o.state_access = 0;
    return o;
}

const char* la_status_string(la_status_t s) {
    int v;  // any integer may arrive: read the bytes, not the enum
    std::memcpy(&v, &s, sizeof v);
    switch (v) {
        case LA_OK: return "ok";
        case LA_ERR_INVALID_ARGUMENT: return "invalid argument";
        case LA_ERR_UNSUPPORTED: return "unsupported configuration";
        case LA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case LA_ERR_HIP: return "HIP launch failed";
        case LA_ERR_WAIT_TIMEOUT: return "a bounded device wait gave up (its rows hold NaN)";
    }
    return "unknown status";
}

size_t la_prefill_workspace_bytes(int32_t Bt, int32_t T, int32_t H, int32_t d, la_dtype_t in_dtype,
                                  la_dtype_t out_dtype, const la_options_t* opt) {
    if (!dtype_arg_ok(in_dtype) || !dtype_arg_ok(out_dtype)) return (size_t)-1;
    Opts o;
    if (Bt < 1 || T < 0 || (int64_t)Bt * T > INT32_MAX) return (size_t)-1;
    if (check_shape(H, d, in_dtype, out_dtype) != LA_OK) return (size_t)-1;
    if (parse_options(opt, H, d, o) != LA_OK || feat_unsupported(o, in_dtype, d)) return (size_t)-1;
    return make_plan(false, Bt, (int64_t)Bt * T, T, H, d, in_dtype, out_dtype, o).total;
}

size_t la_prefill_varlen_workspace_bytes(int32_t total_T, int32_t num_seqs, int32_t max_seqlen,
                                         int32_t H, int32_t d, la_dtype_t in_dtype,
                                         la_dtype_t out_dtype, const la_options_t* opt) {
    if (!dtype_arg_ok(in_dtype) || !dtype_arg_ok(out_dtype)) return (size_t)-1;
    Opts o;
    if (num_seqs < 1 || total_T < 0 || max_seqlen < 0 || max_seqlen > total_T) return (size_t)-1;
    if (check_shape(H, d, in_dtype, out_dtype) != LA_OK) return (size_t)-1;
    if (parse_options(opt, H, d, o) != LA_OK || feat_unsupported(o, in_dtype, d)) return (size_t)-1;
    return make_plan(true, num_seqs, total_T, max_seqlen, H, d, in_dtype, out_dtype, o).total;
}

size_t la_decode_workspace_bytes(int32_t N, int32_t H, int32_t d, la_dtype_t out_dtype,
                                 const la_options_t* opt) {
    if (!dtype_arg_ok(out_dtype)) return (size_t)-1;
    Opts o;
    if (N < 0) return (size_t)-1;
    if (check_shape(H, d, LA_DTYPE_BF16, out_dtype) != LA_OK) return (size_t)-1;
    if (parse_options(opt, H, d, o) != LA_OK) return (size_t)-1;
    if (o.gated && out_dtype != LA_DTYPE_F32) return align256((size_t)N * H * d * sizeof(float));
    return 0;
}

la_status_t la_prefill_plan(int32_t varlen, int32_t num_seqs, int32_t total_T, int32_t max_seqlen,
                            int32_t H, int32_t d, la_dtype_t in_dtype, la_dtype_t out_dtype,
                            int32_t has_state_out, const la_options_t* opt, la_plan_t* plan) {
    if (!dtype_arg_ok(in_dtype) || !dtype_arg_ok(out_dtype)) return LA_ERR_INVALID_ARGUMENT;
    if (!plan) return LA_ERR_INVALID_ARGUMENT;
    if (num_seqs < 1 || total_T < 0 || max_seqlen < 0 || max_seqlen > total_T)
        return LA_ERR_INVALID_ARGUMENT;
    if (!varlen && (int64_t)num_seqs * max_seqlen != total_T) return LA_ERR_INVALID_ARGUMENT;
    la_status_t s = check_shape(H, d, in_dtype, out_dtype);
    if (s != LA_OK) return s;
    Opts o;
    s = parse_options(opt, H, d, o);
    if (s != LA_OK) return s;
    if (feat_unsupported(o, in_dtype, d)) return LA_ERR_UNSUPPORTED;
    const Plan p = make_plan(varlen != 0, num_seqs, total_T, max_seqlen, H, d, in_dtype, out_dtype, o);
    la_plan_t r;
    std::memset(&r, 0, sizeof(r));
    r.main_workgroups = total_T > 0 ? p.items * H : 0;
    r.chunk_tokens = p.C;
    r.block_size = p.block;
    r.fused_gate = total_T > 0 && p.fuse_ok;
    r.chunk_on_device = total_T > 0 && p.cdev;
    int n = 0;
    if (varlen) r.kernels[n++] = LA_KERNEL_CHUNK_TABLE;
    if ((total_T == 0 || (varlen && !p.chunked)) && has_state_out) r.kernels[n++] = LA_KERNEL_STATE_COPY;
    if (total_T > 0) {
        if (p.chunked) {
            r.kernels[n++] = LA_KERNEL_CHUNK_STATE;
            r.kernels[n++] = LA_KERNEL_CHUNK_SCAN;
        }
        if (p.fuse_ok) {
            if (!p.chunked) r.kernels[n++] = LA_KERNEL_EXCHANGE_CLEAR;
            r.kernels[n++] = LA_KERNEL_MAIN_GATED;
        } else {
            r.kernels[n++] = LA_KERNEL_MAIN;
            if (o.gated) r.kernels[n++] = LA_KERNEL_GATE;
        }
    }
    r.n_kernels = n;
    r.status_offset = (total_T > 0 && p.fuse_ok) ? (int64_t)p.off_xbuf : -1;
    *plan = r;
    return LA_OK;
}

la_status_t la_prefill_wait_status(const void* workspace, int64_t status_offset, void* hip_stream) {
    if (status_offset < 0) return LA_OK;
    if (!workspace) return LA_ERR_INVALID_ARGUMENT;
    hipStream_t st = (hipStream_t)hip_stream;
    uint32_t word = 0;
    if (hipMemcpyAsync(&word, (const char*)workspace + status_offset, sizeof word,
                       hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess) {
        (void)hipGetLastError();
        return LA_ERR_HIP;
    }
    return word ? LA_ERR_WAIT_TIMEOUT : LA_OK;
}

la_status_t la_prefill(const void* q, const void* k, const void* v, const void* x_gate,
                       const float* rms_weight, const float* state_in, const float* z_in,
                       void* out, float* state_out, float* z_out, int32_t Bt, int32_t T, int32_t H,
                       int32_t d, la_dtype_t in_dtype, la_dtype_t out_dtype,
                       const la_options_t* opt, void* workspace, size_t workspace_bytes,
                       void* hip_stream) {
    if (!dtype_arg_ok(in_dtype) || !dtype_arg_ok(out_dtype)) return LA_ERR_INVALID_ARGUMENT;
    la_status_t s = check_shape(H, d, in_dtype, out_dtype);
    if (s != LA_OK) return s;
    if (Bt < 1 || T < 0 || (int64_t)Bt * T > INT32_MAX) return LA_ERR_INVALID_ARGUMENT;
    Opts o;
    s = parse_options(opt, H, d, o);
    if (s != LA_OK) return s;
    const int64_t total_T = (int64_t)Bt * T;
    s = check_prefill_common(q, k, v, x_gate, rms_weight, state_in, z_in, out, state_out, z_out, Bt,
                             total_T, H, d, in_dtype, out_dtype, o);
    if (s != LA_OK) return s;
    const Plan p = make_plan(false, Bt, total_T, T, H, d, in_dtype, out_dtype, o);
    s = check_workspace(p, workspace, workspace_bytes);
    if (s != LA_OK) return s;
    return launch_prefill(p, o, in_dtype, out_dtype, q, k, v, x_gate, rms_weight, nullptr, Bt, T,
                          total_T, state_in, z_in, out, state_out, z_out, H, d, (char*)workspace,
                          (hipStream_t)hip_stream);
}

la_status_t la_prefill_noalloc(const void* q, const void* k, const void* v, const void* x_gate,
                               const float* rms_weight, const float* state_in, const float* z_in,
                               void* out, float* state_out, float* z_out, int32_t Bt, int32_t T,
                               int32_t H, int32_t d, la_dtype_t in_dtype, la_dtype_t out_dtype,
                               const la_options_t* opt, void* hip_stream) {
    if (!dtype_arg_ok(in_dtype) || !dtype_arg_ok(out_dtype)) return LA_ERR_INVALID_ARGUMENT;
    la_status_t s = check_shape(H, d, in_dtype, out_dtype);
    if (s != LA_OK) return s;
    if (Bt < 1 || T < 0 || (int64_t)Bt * T > INT32_MAX) return LA_ERR_INVALID_ARGUMENT;
    Opts o;
    s = parse_options(opt, H, d, o);
    if (s != LA_OK) return s;
    const int64_t total_T = (int64_t)Bt * T;
    s = check_prefill_common(q, k, v, x_gate, rms_weight, state_in, z_in, out, state_out, z_out, Bt,
                             total_T, H, d, in_dtype, out_dtype, o);
    if (s != LA_OK) return s;
    Plan p = make_plan(false, Bt, total_T, T, H, d, in_dtype, out_dtype, o);
    // the half-chunk state pass needs room for its partial increments: without
    // it the plan may still fit the array
    if (p.total > (size_t)LA_NOALLOC_SCRATCH_BYTES && p.half)
        p = make_plan(false, Bt, total_T, T, H, d, in_dtype, out_dtype, o, false);
    if (p.total > (size_t)LA_NOALLOC_SCRATCH_BYTES) return LA_ERR_WORKSPACE_TOO_SMALL;
    void* ws = nullptr;
    if (p.total > 0) {
        ws = scratch_for_current_device();
        if (!ws) return LA_ERR_HIP;
    }
    return launch_prefill(p, o, in_dtype, out_dtype, q, k, v, x_gate, rms_weight, nullptr, Bt, T,
                          total_T, state_in, z_in, out, state_out, z_out, H, d, (char*)ws,
                          (hipStream_t)hip_stream);
}

// Validation, then (launch) the kernels: with launch = false a call is only
// checked, so that a serving step can check both of its parts first.
static la_status_t prefill_varlen_impl(bool launch, const void* q, const void* k, const void* v,
                                       const void* x_gate, const float* rms_weight,
                                       const int32_t* cu_seqlens, int32_t num_seqs, int32_t total_T,
                                       int32_t max_seqlen, const float* state_in, const float* z_in,
                                       void* out, float* state_out, float* z_out, int32_t H, int32_t d,
                                       la_dtype_t in_dtype, la_dtype_t out_dtype,
                                       const la_options_t* opt, void* workspace,
                                       size_t workspace_bytes, void* hip_stream) {
    la_status_t s = check_shape(H, d, in_dtype, out_dtype);
    if (s != LA_OK) return s;
    if (!cu_seqlens || !aligned(cu_seqlens, 4) || num_seqs < 1 || total_T < 0 || max_seqlen < 0 ||
        max_seqlen > total_T)
        return LA_ERR_INVALID_ARGUMENT;
    Opts o;
    s = parse_options(opt, H, d, o);
    if (s != LA_OK) return s;
    s = check_prefill_common(q, k, v, x_gate, rms_weight, state_in, z_in, out, state_out, z_out,
                             num_seqs, total_T, H, d, in_dtype, out_dtype, o);
    if (s != LA_OK) return s;
    const Plan p = make_plan(true, num_seqs, total_T, max_seqlen, H, d, in_dtype, out_dtype, o);
    s = check_workspace(p, workspace, workspace_bytes);
    if (s != LA_OK || !launch) return s;
    return launch_prefill(p, o, in_dtype, out_dtype, q, k, v, x_gate, rms_weight, cu_seqlens,
                          num_seqs, 0, total_T, state_in, z_in, out, state_out, z_out, H, d,
                          (char*)workspace, (hipStream_t)hip_stream);
}

la_status_t la_prefill_varlen(const void* q, const void* k, const void* v, const void* x_gate,
                              const float* rms_weight, const int32_t* cu_seqlens, int32_t num_seqs,
                              int32_t total_T, int32_t max_seqlen, const float* state_in,
                              const float* z_in, void* out, float* state_out, float* z_out,
                              int32_t H, int32_t d, la_dtype_t in_dtype, la_dtype_t out_dtype,
                              const la_options_t* opt, void* workspace, size_t workspace_bytes,
                              void* hip_stream) {
    if (!dtype_arg_ok(in_dtype) || !dtype_arg_ok(out_dtype)) return LA_ERR_INVALID_ARGUMENT;
    return prefill_varlen_impl(true, q, k, v, x_gate, rms_weight, cu_seqlens, num_seqs, total_T,
                               max_seqlen, state_in, z_in, out, state_out, z_out, H, d, in_dtype,
                               out_dtype, opt, workspace, workspace_bytes, hip_stream);
}

static la_status_t decode_step_impl(bool launch, const void* q, const void* k, const void* v,
                                    const void* x_gate, const float* rms_weight, float* state,
                                    float* z, void* out, int32_t N, int32_t H, int32_t d,
                                    la_dtype_t in_dtype, la_dtype_t out_dtype,
                                    const la_options_t* opt, void* workspace,
                                    size_t workspace_bytes, void* hip_stream) {
    la_status_t s = check_shape(H, d, in_dtype, out_dtype);
    if (s != LA_OK) return s;
    if (N < 0) return LA_ERR_INVALID_ARGUMENT;
    Opts o;
    s = parse_options(opt, H, d, o);
    if (s != LA_OK) return s;
    if (!q || !k || !v || !state || !out) return LA_ERR_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(state, 16) || !aligned(out, 16))
        return LA_ERR_INVALID_ARGUMENT;
    if (o.normalized && (!z || !aligned(z, 16))) return LA_ERR_INVALID_ARGUMENT;
    if (!o.normalized && z) return LA_ERR_INVALID_ARGUMENT;
    if (o.gated && (!x_gate || !aligned(x_gate, 16))) return LA_ERR_INVALID_ARGUMENT;
    if (rms_weight && !aligned(rms_weight, 16)) return LA_ERR_INVALID_ARGUMENT;
    const size_t in_bytes = (size_t)N * H * d * dtype_size(in_dtype);
    const size_t out_bytes = (size_t)N * H * d * dtype_size(out_dtype);
    const int64_t srows = o.slots ? o.rows : N;  // rows of state and z
    const size_t s_bytes = (size_t)srows * H * d * d * sizeof(float);
    const void* ins[4] = {q, k, v, o.gated ? x_gate : nullptr};
    for (const void* ip : ins) {
        if (overlap(out, out_bytes, ip, in_bytes)) return LA_ERR_INVALID_ARGUMENT;
        if (overlap(state, s_bytes, ip, in_bytes)) return LA_ERR_INVALID_ARGUMENT;
    }
    if (overlap(out, out_bytes, state, s_bytes)) return LA_ERR_INVALID_ARGUMENT;
    if (z && (overlap(out, out_bytes, z, (size_t)srows * H * d * 4) || overlap(state, s_bytes, z, (size_t)srows * H * d * 4)))
        return LA_ERR_INVALID_ARGUMENT;
    const size_t need = (o.gated && out_dtype != LA_DTYPE_F32) ? align256((size_t)N * H * d * sizeof(float)) : 0;
    if (need) {
        if (!workspace || !aligned(workspace, 256)) return LA_ERR_INVALID_ARGUMENT;
        if (workspace_bytes < need) return LA_ERR_WORKSPACE_TOO_SMALL;
    }
    if (N == 0 || !launch) return LA_OK;
    hipStream_t st = (hipStream_t)hip_stream;
    Timer tm(o, st);
    void* ydst = o.gated ? (need ? workspace : out) : out;
    const bool yf32 = o.gated || out_dtype == LA_DTYPE_F32;
    // The state's access mode: streaming (non-temporal hints, one workgroup
    // per (sequence, head) streaming its block contiguously) unless the state
    // the call touches is small enough to stay cache-resident between calls
    // (auto: under a quarter of the 256 MB Infinity Cache; a serving step
    // streams every layer's state and weights between two visits to one
    // layer), or the caller says it is.  Cache-resident, plain mode, d = 128:
    // kDecodeSplit workgroups per (sequence, head), each owning 128 /
    // kDecodeSplit state columns.
    const int64_t touched = (int64_t)N * H * d * d * 4;
    const bool stream = o.state_access == 1 || (o.state_access == 0 && touched >= kStreamStateBytes);
    const unsigned grid = (unsigned)((int64_t)N * H);
#define LA_DEC(DD, IT, OT, NN)                                                                     \
    do {                                                                                           \
        if (stream) {                                                                              \
            k_decode<DD, IT, OT, NN, 1, true><<<grid, 256, 0, st>>>((const IT*)q, (const IT*)k,     \
                (const IT*)v, state, z, (OT*)ydst, o.slots, o.rows, H, o.feat ? 1 : 0);           \
        } else {                                                                                   \
            constexpr int SP = (!(NN) && (DD) == 128) ? kDecodeSplit : 1;                          \
            k_decode<DD, IT, OT, NN, SP><<<grid * SP, 256, 0, st>>>((const IT*)q, (const IT*)k,     \
                (const IT*)v, state, z, (OT*)ydst, o.slots, o.rows, H, o.feat ? 1 : 0);           \
        }                                                                                          \
    } while (0)
#define LA_DEC_OUT(DD, IT)                                                                  \
    do {                                                                                    \
        if (yf32) { if (o.normalized) LA_DEC(DD, IT, float, true); else LA_DEC(DD, IT, float, false); } \
        else { if (o.normalized) LA_DEC(DD, IT, uint16_t, true); else LA_DEC(DD, IT, uint16_t, false); } \
    } while (0)
    tm.before();
    if (in_dtype == LA_DTYPE_BF16) {
        if (d == 128) LA_DEC_OUT(128, uint16_t); else LA_DEC_OUT(64, uint16_t);
    } else {
        if (d == 128) LA_DEC_OUT(128, float); else LA_DEC_OUT(64, float);
    }
#undef LA_DEC_OUT
#undef LA_DEC
    if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
    tm.after();
    if (o.gated) {
        const int F = H * d;
        const int64_t units = (int64_t)N * (F / o.group);
        const unsigned blocks = (unsigned)((units + 3) / 4);
        const float* yf = (const float*)ydst;
        tm.before();
#define LA_GATE(XT, OT)                                                                                     \
    do {                                                                                                    \
        launch_gate<XT, OT>(blocks, st, yf, (const XT*)x_gate, rms_weight, (OT*)out, N, F, o.group, o.eps); \
    } while (0)
        if (in_dtype == LA_DTYPE_BF16) {
            if (out_dtype == LA_DTYPE_BF16) LA_GATE(uint16_t, uint16_t); else LA_GATE(uint16_t, float);
        } else {
            if (out_dtype == LA_DTYPE_BF16) LA_GATE(float, uint16_t); else LA_GATE(float, float);
        }
#undef LA_GATE
        if (hipGetLastError() != hipSuccess) return LA_ERR_HIP;
        tm.after();
    }
    return LA_OK;
}

la_status_t la_decode_step(const void* q, const void* k, const void* v, const void* x_gate,
                           const float* rms_weight, float* state, float* z, void* out, int32_t N,
                           int32_t H, int32_t d, la_dtype_t in_dtype, la_dtype_t out_dtype,
                           const la_options_t* opt, void* workspace, size_t workspace_bytes,
                           void* hip_stream) {
    if (!dtype_arg_ok(in_dtype) || !dtype_arg_ok(out_dtype)) return LA_ERR_INVALID_ARGUMENT;
    return decode_step_impl(true, q, k, v, x_gate, rms_weight, state, z, out, N, H, d, in_dtype,
                            out_dtype, opt, workspace, workspace_bytes, hip_stream);
}

// ------------------------------------------------------------- serving --

la_status_t la_schedule_step(const la_request_t* reqs, int32_t R, int32_t max_batched_tokens,
                             int32_t* order, int32_t* chunk, la_step_t* step) {
    if (R < 0 || !step || (R > 0 && (!reqs || !order || !chunk))) return LA_ERR_INVALID_ARGUMENT;
    int32_t nd = 0;
    for (int32_t r = 0; r < R; ++r) {
        if (reqs[r].remaining < 0) return LA_ERR_INVALID_ARGUMENT;
        if (reqs[r].remaining == 0) ++nd;
    }
    if (max_batched_tokens < nd) return LA_ERR_INVALID_ARGUMENT;
    la_step_t st{};
    int32_t n = 0;
    for (int32_t r = 0; r < R; ++r) {
        if (reqs[r].remaining == 0) {
            order[n] = r;
            chunk[n] = 1;
            ++n;
        }
    }
    st.num_decode = n;
    int64_t budget = (int64_t)max_batched_tokens - n;
    for (int32_t r = 0; r < R && budget > 0; ++r) {
        if (reqs[r].remaining == 0) continue;
        const int32_t c = (int32_t)(reqs[r].remaining < budget ? reqs[r].remaining : budget);
        order[n] = r;
        chunk[n] = c;
        ++n;
        ++st.num_prefill;
        st.prefill_tokens += c;
        if (c > st.max_chunk) st.max_chunk = c;
        budget -= c;
    }
    *step = st;
    return LA_OK;
}

namespace {

// Workspace split of a serving step: [decode part | prefill part], each
// 256-byte aligned.
struct ServeWs {
    size_t dec, pre, total;
};

ServeWs serve_ws(int32_t num_decode, int32_t num_prefill, int32_t prefill_tokens,
                 int32_t max_chunk, int32_t H, int32_t d, la_dtype_t in_dtype,
                 la_dtype_t out_dtype, const la_options_t* opt) {
    ServeWs w{0, 0, (size_t)-1};
    const size_t a = num_decode > 0 ? la_decode_workspace_bytes(num_decode, H, d, out_dtype, opt) : 0;
    const size_t b = num_prefill > 0
                         ? la_prefill_varlen_workspace_bytes(prefill_tokens, num_prefill, max_chunk, H,
                                                             d, in_dtype, out_dtype, opt)
                         : 0;
    if (a == (size_t)-1 || b == (size_t)-1) return w;
    w.dec = align256(a);
    w.pre = align256(b);
    w.total = w.dec + w.pre;
    return w;
}

}  // namespace

size_t la_serve_step_workspace_bytes(int32_t num_decode, int32_t num_prefill,
                                     int32_t prefill_tokens, int32_t max_chunk, int32_t H,
                                     int32_t d, la_dtype_t in_dtype, la_dtype_t out_dtype,
                                     const la_options_t* opt) {
    if (!dtype_arg_ok(in_dtype) || !dtype_arg_ok(out_dtype)) return (size_t)-1;
    if (num_decode < 0 || num_prefill < 0 || prefill_tokens < 0) return (size_t)-1;
    return serve_ws(num_decode, num_prefill, prefill_tokens, max_chunk, H, d, in_dtype, out_dtype,
                    opt).total;
}

la_status_t la_serve_step(const void* q, const void* k, const void* v, const void* x_gate,
                          const float* rms_weight, float* state_pool, float* z_pool,
                          int32_t state_rows, const int32_t* decode_slots, int32_t num_decode,
                          const int32_t* prefill_cu, const int32_t* prefill_slots,
                          int32_t num_prefill, int32_t prefill_tokens, int32_t max_chunk,
                          void* out, int32_t H, int32_t d, la_dtype_t in_dtype,
                          la_dtype_t out_dtype, const la_options_t* opt, void* workspace,
                          size_t workspace_bytes, void* decode_stream, void* prefill_stream) {
    if (!dtype_arg_ok(in_dtype) || !dtype_arg_ok(out_dtype)) return LA_ERR_INVALID_ARGUMENT;
    la_status_t s = check_shape(H, d, in_dtype, out_dtype);
    if (s != LA_OK) return s;
    if (num_decode < 0 || num_prefill < 0 || prefill_tokens < 0 || state_rows < 1 || !state_pool)
        return LA_ERR_INVALID_ARGUMENT;
    if ((num_decode > 0 && !decode_slots) || (num_prefill > 0 && (!prefill_slots || !prefill_cu)))
        return LA_ERR_INVALID_ARGUMENT;
    if (num_prefill == 0 && prefill_tokens != 0) return LA_ERR_INVALID_ARGUMENT;
    if (num_prefill > 0 && (max_chunk < 1 || max_chunk > prefill_tokens)) return LA_ERR_INVALID_ARGUMENT;
    const la_options_t base = opt ? *opt : la_default_options();
    if (base.state_slots) return LA_ERR_INVALID_ARGUMENT;  // the slots are arguments here
    const ServeWs w = serve_ws(num_decode, num_prefill, prefill_tokens, max_chunk, H, d, in_dtype,
                               out_dtype, &base);
    if (w.total == (size_t)-1) return LA_ERR_INVALID_ARGUMENT;
    if (w.total) {
        if (!workspace || !aligned(workspace, 256)) return LA_ERR_INVALID_ARGUMENT;
        if (workspace_bytes < w.total) return LA_ERR_WORKSPACE_TOO_SMALL;
    }
    // both parts are checked before either is enqueued: a rejected step has no side effects
    const size_t isz = dtype_size(in_dtype), osz = dtype_size(out_dtype);
    const size_t row_in = (size_t)H * d * isz, row_out = (size_t)H * d * osz;
    la_options_t od = base, op = base;
    od.state_slots = decode_slots;
    od.state_rows = state_rows;
    op.state_slots = prefill_slots;
    op.state_rows = state_rows;
    od.timing_events = op.timing_events = nullptr;
    od.n_timing = op.n_timing = 0;
    char* ws = (char*)workspace;
    const char* qb = (const char*)q + (size_t)num_decode * row_in;
    const char* kb = (const char*)k + (size_t)num_decode * row_in;
    const char* vb = (const char*)v + (size_t)num_decode * row_in;
    const char* xb = x_gate ? (const char*)x_gate + (size_t)num_decode * row_in : nullptr;
    char* ob = (char*)out + (size_t)num_decode * row_out;
    for (int pass = 0; pass < 2; ++pass) {
        const bool launch = pass == 1;
        if (num_decode > 0) {
            s = decode_step_impl(launch, q, k, v, x_gate, rms_weight, state_pool, z_pool, out,
                                 num_decode, H, d, in_dtype, out_dtype, &od, w.dec ? ws : nullptr,
                                 w.dec, decode_stream);
            if (s != LA_OK) return s;
        }
        if (num_prefill > 0) {
            s = prefill_varlen_impl(launch, qb, kb, vb, xb, rms_weight, prefill_cu, num_prefill,
                                    prefill_tokens, max_chunk, state_pool, z_pool, ob, state_pool,
                                    z_pool, H, d, in_dtype, out_dtype, &op, w.pre ? ws + w.dec : nullptr,
                                    w.pre, prefill_stream);
            if (s != LA_OK) return s;
        }
    }
    return LA_OK;
}

}  // extern "C"
