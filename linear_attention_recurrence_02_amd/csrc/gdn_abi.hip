// libgdn C ABI: argument validation and launch selection (see include/gdn.h).
// Nothing here allocates device memory or synchronises (except the opt-in
// debugging check of packed offsets below); a rejected call enqueues nothing.

#include "gdn.h"
#include "gdn_internal.hpp"

#include <atomic>
#include <cfloat>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 31;

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
};

Range span_of(const void *p, int64_t bytes) {
    uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + static_cast<uintptr_t>(bytes)};
}

bool overlap(Range a, Range b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool dims_ok(int64_t x) { return x >= 0 && x < kMaxDim; }

// Opt-in debugging check of packed offsets: with GDN_CHECK_SEQLENS set (to
// anything but "0"), cu_seqlens is copied to the host on the caller's stream,
// which is then synchronised, and must start at 0, never decrease and end at
// T.  Without it the kernels read the offsets on the device and clamp them.
int check_seqlens_debug(const int32_t *cu, int64_t N, int64_t T, void *stream) {
    const char *env = std::getenv("GDN_CHECK_SEQLENS");
    if (!cu || !env || !*env || std::strcmp(env, "0") == 0) return GDN_OK;
    std::vector<int32_t> h(static_cast<size_t>(N) + 1);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(h.data(), cu, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s) !=
            hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return GDN_ERR_HIP;
    if (h[0] != 0 || h[static_cast<size_t>(N)] != T) return GDN_ERR_INVALID_ARG;
    for (int64_t n = 0; n < N; ++n)
        if (h[static_cast<size_t>(n) + 1] < h[static_cast<size_t>(n)]) return GDN_ERR_INVALID_ARG;
    return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_version(void) { return 1; }

const char *gdn_status_string(int status) {
    switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_INVALID_ARG: return "invalid argument (null pointer, bad size or misaligned buffer)";
    case GDN_ERR_UNSUPPORTED: return "unsupported configuration (dk/dv must be 128, chunk 16/32/64, dtype f32/bf16)";
    case GDN_ERR_ALIAS: return "buffers overlap in a way the call forbids";
    case GDN_ERR_HIP: return "HIP runtime error while enqueuing a kernel";
    case GDN_ERR_SCRATCH: return "the call needs more scratch than the no-allocation entry point holds";
    default: return "unknown status";
    }
}

}  // extern "C"

int gdn::compute_units() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return 0;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

namespace {

// Validation shared by the prompt-form calls: fills `a` (and the byte spans
// of the token buffers for further alias checks) or returns a status.
// GDN_BF16_F32_OUT (bf16 inputs, fp32 O) only where `f32_out_ok`.
int check_prefill(const void *q, const void *k, const void *v, int io_dtype, const float *g,
                  const float *beta, const float *S0, const int32_t *cu_seqlens,
                  int64_t B_or_N, int64_t T, int64_t H, int64_t dk, int64_t dv,
                  int64_t chunk, void *O, float *S_T, gdn::PrefillArgs &a, int64_t &tok_bytes,
                  bool f32_out_ok = false) {
    if (!dims_ok(B_or_N) || !dims_ok(T) || H <= 0 || H >= 65536) return GDN_ERR_INVALID_ARG;
    const int64_t N = B_or_N;
    const int64_t rows = cu_seqlens ? T : N * T;        // token rows of H heads
    // Token buffers may be NULL only when the call has no token rows at all.
    if (rows > 0 && (!q || !k || !v || !g || !beta || !O)) return GDN_ERR_INVALID_ARG;
    if (!S_T) return GDN_ERR_INVALID_ARG;
    const bool f32_out = io_dtype == GDN_BF16_F32_OUT;
    if (io_dtype != GDN_F32 && io_dtype != GDN_BF16 && !(f32_out && f32_out_ok))
        return GDN_ERR_UNSUPPORTED;
    if (dk != gdn::kHeadDim || dv != gdn::kHeadDim) return GDN_ERR_UNSUPPORTED;
    if (chunk != 16 && chunk != 32 && chunk != 64) return GDN_ERR_UNSUPPORTED;
    for (const void *p : {q, k, v, static_cast<const void *>(O)})
        if (!aligned(p, 16)) return GDN_ERR_INVALID_ARG;
    if (!aligned(S_T, 16) || (S0 && !aligned(S0, 16))) return GDN_ERR_INVALID_ARG;
    if (!aligned(g, 4) || !aligned(beta, 4) || (cu_seqlens && !aligned(cu_seqlens, 4)))
        return GDN_ERR_INVALID_ARG;

    if (N * H >= kMaxDim) return GDN_ERR_INVALID_ARG;     // one workgroup per unit
    if (rows > (int64_t(1) << 40) / (H * gdn::kHeadDim)) return GDN_ERR_INVALID_ARG;
    const int64_t esz = io_dtype == GDN_F32 ? 4 : 2;
    tok_bytes = rows * H * gdn::kHeadDim * esz;
    const int64_t out_bytes = f32_out ? 2 * tok_bytes : tok_bytes;
    const int64_t gb_bytes = rows * H * 4;
    const int64_t st_bytes = N * H * gdn::kHeadDim * gdn::kHeadDim * 4;

    const Range rq = span_of(q, tok_bytes), rk = span_of(k, tok_bytes),
                rv = span_of(v, tok_bytes), rg = span_of(g, gb_bytes),
                rb = span_of(beta, gb_bytes), rO = span_of(O, out_bytes),
                rST = span_of(S_T, st_bytes),
                rS0 = S0 ? span_of(S0, st_bytes) : Range{0, 0};
    for (Range r : {rq, rk, rv, rg, rb, rS0, rST})
        if (overlap(rO, r)) return GDN_ERR_ALIAS;
    for (Range r : {rq, rk, rv, rg, rb})
        if (overlap(rST, r)) return GDN_ERR_ALIAS;
    if (S0 && overlap(rST, rS0) && rST.lo != rS0.lo) return GDN_ERR_ALIAS;

    a = gdn::PrefillArgs{q, k, v, g, beta, S0, cu_seqlens, N, T, H,
                         static_cast<int>(chunk), io_dtype != GDN_F32, O, S_T};
    a.out_f32 = f32_out;
    return GDN_OK;
}

int launch_prefill(const gdn::PrefillArgs &a, void *stream) {
    if (a.N == 0) return GDN_OK;   // nothing to do
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = gdn::prefill_short_pays(a)     ? gdn::launch_prefill_short(a, s)
                   : gdn::prefill_mfma_supports(a) ? gdn::launch_prefill_mfma(a, s)
                                                   : gdn::launch_prefill_valu(a, s);
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

// Workspace of the segmented prompt form: the segments' offsets, each
// sequence's first segment, and three arrays of one state per (segment,
// head).  A uniform batch has N ceil(T / L) segments (at least N); a packed one
// at most N + ceil(T / L), each sequence rounding up once.  Parts are 256-byte
// aligned; false for sizes it cannot hold.
struct SegLayout {
    int64_t Ns, rows, cu, seg, s1, m, b, total;
};

bool seg_layout(int io_dtype, bool packed, int64_t N, int64_t T, int64_t H, int64_t L,
                SegLayout &w) {
    if (!dims_ok(N) || !dims_ok(T) || H <= 0 || H >= 65536 || L <= 0) return false;
    if (io_dtype != GDN_F32 && io_dtype != GDN_BF16) return false;
    const int64_t per = (T + L - 1) / L;
    w.rows = packed ? T : N * T;
    if (w.rows >= kMaxDim) return false;           // the segments' offsets are int32
    w.Ns = packed ? N + per : N * (per > 0 ? per : 1);
    const int64_t units = w.Ns * H;
    if (w.Ns >= kMaxDim || units >= kMaxDim) return false;
    if (w.rows > (int64_t(1) << 40) / (H * gdn::kHeadDim)) return false;
    auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
    const int64_t state = gdn::kHeadDim * gdn::kHeadDim * 4;
    w.cu = 0;
    w.seg = up((w.Ns + 1) * 4);
    w.s1 = w.seg + up((N + 1) * 4);
    w.m = w.s1 + up(units * state);
    w.b = w.m + up(units * state);
    w.total = w.b + up(units * state);
    return true;
}

// The segmented form on a validated call, with its workspace at `ws` (at
// least w.total bytes, 256-byte aligned, disjoint from the call's buffers).
int run_segmented(const gdn::PrefillArgs &a, const SegLayout &w, char *ws, int64_t segment_len,
                  void *stream) {
    const int64_t N = a.N, H = a.H;
    int32_t *cu = reinterpret_cast<int32_t *>(ws + w.cu);    // the segments' offsets
    int32_t *seg = reinterpret_cast<int32_t *>(ws + w.seg);  // each sequence's first segment
    float *s1 = reinterpret_cast<float *>(ws + w.s1);   // identity states, then S_in
    float *m = reinterpret_cast<float *>(ws + w.m);     // state maps
    float *b = reinterpret_cast<float *>(ws + w.b);     // zero-start states, then end states
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto run = [&](const void *vv, const float *s0, void *O, float *st_out) {
        gdn::PrefillArgs r = a;
        r.v = vv;
        r.S0 = s0;
        r.O = O;
        r.S_T = st_out;
        r.cu_seqlens = cu;
        r.N = w.Ns;
        r.T = w.rows;
        return launch_prefill(r, stream);
    };
    if (gdn::launch_segment_prep(a.cu_seqlens, N, a.T, segment_len, w.Ns, seg, cu, s1, w.Ns * H, s) !=
        hipSuccess)
        return GDN_ERR_HIP;
    int rc = run(a.v, nullptr, nullptr, b);            // B: each segment from zero, no O
    if (rc == GDN_OK) rc = run(nullptr, s1, nullptr, m);   // M: no values, from the identity
    if (rc != GDN_OK) return rc;
    if (gdn::launch_segment_scan(m, b, a.S0, s1, seg, N, H, s) != hipSuccess) return GDN_ERR_HIP;
    rc = run(a.v, s1, a.O, b);                         // O and the end states from S_in
    if (rc != GDN_OK) return rc;
    return gdn::launch_segment_gather(b, a.S0, seg, a.S_T, N, H, s) == hipSuccess ? GDN_OK
                                                                                   : GDN_ERR_HIP;
}

// Validation shared by the two segmented entry points: fills `a` and `w`;
// GDN_OK with w.total == 0 means the call is the plain form (launched here).
int check_segmented(const void *q, const void *k, const void *v, int io_dtype, const float *g,
                    const float *beta, const float *S0, const int32_t *cu_seqlens, int64_t B_or_N,
                    int64_t T, int64_t H, int64_t dk, int64_t dv, int64_t chunk,
                    int64_t segment_len, void *O, float *S_T, void *stream, gdn::PrefillArgs &a,
                    SegLayout &w, int64_t &tok_bytes, bool &done) {
    done = false;
    const int st = check_prefill(q, k, v, io_dtype, g, beta, S0, cu_seqlens, B_or_N, T, H, dk,
                                 dv, chunk, O, S_T, a, tok_bytes);
    if (st != GDN_OK) return st;
    if (segment_len <= 0 || segment_len % chunk != 0) return GDN_ERR_INVALID_ARG;
    if (!seg_layout(io_dtype, cu_seqlens != nullptr, B_or_N, T, H, segment_len, w))
        return GDN_ERR_INVALID_ARG;
    if (const int sc = check_seqlens_debug(cu_seqlens, B_or_N, T, stream)) return sc;
    // a uniform batch of one segment per sequence is the plain form
    if (B_or_N == 0 || (!cu_seqlens && T <= segment_len)) {
        done = true;
        return launch_prefill(a, stream);
    }
    return GDN_OK;
}

// Whether the byte range [p, p + bytes) overlaps any buffer of the call.
bool overlaps_call(const void *p, int64_t bytes, const gdn::PrefillArgs &a, int64_t tok_bytes) {
    const int64_t gb = (a.cu_seqlens ? a.T : a.N * a.T) * a.H * 4,
                  st_bytes = a.N * a.H * gdn::kHeadDim * gdn::kHeadDim * 4;
    const Range rw = span_of(p, bytes);
    for (Range r : {span_of(a.q, tok_bytes), span_of(a.k, tok_bytes), span_of(a.v, tok_bytes),
                    span_of(a.g, gb), span_of(a.beta, gb), span_of(a.O, tok_bytes),
                    span_of(a.S_T, st_bytes), a.S0 ? span_of(a.S0, st_bytes) : Range{0, 0},
                    a.cu_seqlens ? span_of(a.cu_seqlens, (a.N + 1) * 4) : Range{0, 0}})
        if (overlap(rw, r)) return true;
    return false;
}

// Scratch of the no-allocation segmented form: a file-scope device array,
// one copy per GPU, held while the library is loaded.  Host code uses the
// address hipGetSymbolAddress returns for the current device, never the
// array's name (which on the host is only a stand-in).
constexpr int64_t kNoAllocScratchBytes = (int64_t(48) << 20) + (int64_t(64) << 10);
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// The current device's address of `scratch`, looked up once per device.
char *scratch_address() {
    static std::mutex mu;
    static char *addr[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        addr[dev] = static_cast<char *>(p);
    }
    return addr[dev];
}

}  // namespace

extern "C" {

int64_t gdn_chunk_prefill_segmented_workspace(int io_dtype, const int32_t *cu_seqlens,
                                              int64_t B_or_N, int64_t T, int64_t H,
                                              int64_t segment_len) {
    SegLayout w;
    return seg_layout(io_dtype, cu_seqlens != nullptr, B_or_N, T, H, segment_len, w) ? w.total
                                                                                      : -1;
}

int gdn_chunk_prefill_segmented(const void *q, const void *k, const void *v, int io_dtype,
                                const float *g, const float *beta, const float *S0,
                                const int32_t *cu_seqlens, int64_t B_or_N, int64_t T, int64_t H,
                                int64_t dk, int64_t dv, int64_t chunk, int64_t segment_len,
                                void *workspace, int64_t workspace_bytes, void *O, float *S_T,
                                void *stream) {
    gdn::PrefillArgs a{};
    SegLayout w{};
    int64_t tok_bytes = 0;
    bool done = false;
    const int st = check_segmented(q, k, v, io_dtype, g, beta, S0, cu_seqlens, B_or_N, T, H, dk,
                                   dv, chunk, segment_len, O, S_T, stream, a, w, tok_bytes, done);
    if (st != GDN_OK || done) return st;
    if (!workspace || workspace_bytes < w.total || !aligned(workspace, 256))
        return GDN_ERR_INVALID_ARG;
    if (overlaps_call(workspace, w.total, a, tok_bytes)) return GDN_ERR_ALIAS;
    return run_segmented(a, w, static_cast<char *>(workspace), segment_len, stream);
}

int gdn_chunk_prefill_segmented_noalloc(const void *q, const void *k, const void *v, int io_dtype,
                                        const float *g, const float *beta, const float *S0,
                                        const int32_t *cu_seqlens, int64_t B_or_N, int64_t T,
                                        int64_t H, int64_t dk, int64_t dv, int64_t chunk,
                                        int64_t segment_len, void *O, float *S_T, void *stream) {
    gdn::PrefillArgs a{};
    SegLayout w{};
    int64_t tok_bytes = 0;
    bool done = false;
    const int st = check_segmented(q, k, v, io_dtype, g, beta, S0, cu_seqlens, B_or_N, T, H, dk,
                                   dv, chunk, segment_len, O, S_T, stream, a, w, tok_bytes, done);
    if (st != GDN_OK || done) return st;
    if (w.total > kNoAllocScratchBytes) return GDN_ERR_SCRATCH;
    char *ws = scratch_address();
    if (!ws) return GDN_ERR_HIP;
    return run_segmented(a, w, ws, segment_len, stream);
}

int64_t gdn_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

int gdn_chunk_prefill(const void *q, const void *k, const void *v, int io_dtype,
                      const float *g, const float *beta, const float *S0,
                      const int32_t *cu_seqlens, int64_t B_or_N, int64_t T,
                      int64_t H, int64_t dk, int64_t dv, int64_t chunk, void *O,
                      float *S_T, void *stream) {
    gdn::PrefillArgs a{};
    int64_t tok_bytes = 0;
    const int st = check_prefill(q, k, v, io_dtype, g, beta, S0, cu_seqlens, B_or_N, T, H, dk,
                                 dv, chunk, O, S_T, a, tok_bytes, true);
    if (st != GDN_OK) return st;
    if (const int sc = check_seqlens_debug(cu_seqlens, B_or_N, T, stream)) return sc;
    return launch_prefill(a, stream);
}

int gdn_chunk_prefill_ex(const void *q, const void *k, const void *v, int io_dtype,
                         const float *g, const float *beta, const float *S0,
                         const int32_t *cu_seqlens, int64_t B_or_N, int64_t T, int64_t H,
                         int64_t dk, int64_t dv, int64_t chunk, int inverse, int columns,
                         void *O, float *S_T, void *stream) {
    if (inverse != GDN_INVERSE_DEFAULT && inverse != GDN_INVERSE_SUBSTITUTION &&
        inverse != GDN_INVERSE_DOUBLING)
        return GDN_ERR_UNSUPPORTED;
    if (columns != GDN_COLUMNS_DEFAULT && columns != GDN_COLUMNS_WHOLE &&
        columns != GDN_COLUMNS_SPLIT)
        return GDN_ERR_UNSUPPORTED;
    gdn::PrefillArgs a{};
    int64_t tok_bytes = 0;
    const int st = check_prefill(q, k, v, io_dtype, g, beta, S0, cu_seqlens, B_or_N, T, H, dk,
                                 dv, chunk, O, S_T, a, tok_bytes, true);
    if (st != GDN_OK) return st;
    if (const int sc = check_seqlens_debug(cu_seqlens, B_or_N, T, stream)) return sc;
    if (inverse != GDN_INVERSE_DEFAULT) {
        a.inverse = inverse == GDN_INVERSE_DOUBLING ? gdn::kInverseDoubling
                                                    : gdn::kInverseSubstitution;
        a.short_ok = false;
    }
    if (columns != GDN_COLUMNS_DEFAULT) {
        a.columns = columns == GDN_COLUMNS_SPLIT ? gdn::kColumnsSplit : gdn::kColumnsWhole;
        a.short_ok = false;
    }
    return launch_prefill(a, stream);
}

int gdn_chunk_prefill_gated(const void *q, const void *k, const void *v, int io_dtype,
                            const float *g, const float *beta, const float *S0,
                            const int32_t *cu_seqlens, int64_t B_or_N, int64_t T,
                            int64_t H, int64_t dk, int64_t dv, int64_t chunk,
                            const void *z, const float *norm_w, float eps, void *Y,
                            float *S_T, void *stream) {
    gdn::PrefillArgs a{};
    int64_t tok_bytes = 0;
    const int st = check_prefill(q, k, v, io_dtype, g, beta, S0, cu_seqlens, B_or_N, T, H, dk,
                                 dv, chunk, Y, S_T, a, tok_bytes);
    if (st != GDN_OK) return st;
    if (!norm_w || !aligned(norm_w, 4)) return GDN_ERR_INVALID_ARG;
    if (tok_bytes > 0 && !z) return GDN_ERR_INVALID_ARG;
    if (!aligned(z, 16)) return GDN_ERR_INVALID_ARG;
    if (!(eps >= 0.f && eps <= FLT_MAX)) return GDN_ERR_INVALID_ARG;   // finite, >= 0
    const Range rz = span_of(z, tok_bytes), rw = span_of(norm_w, gdn::kHeadDim * 4),
                rY = span_of(Y, tok_bytes),
                rST = span_of(S_T, a.N * H * gdn::kHeadDim * gdn::kHeadDim * 4);
    for (Range r : {rz, rw})
        if (overlap(rY, r) || overlap(rST, r)) return GDN_ERR_ALIAS;
    if (const int sc = check_seqlens_debug(cu_seqlens, B_or_N, T, stream)) return sc;
    // z is NULL only in a call without token rows, where the plain form does
    // the same work (S_T = S0)
    a.z = z;
    a.norm_w = norm_w;
    a.eps = eps;
    return launch_prefill(a, stream);
}

int gdn_prefill_states(const void *q, const void *k, const void *v, int io_dtype,
                       const float *g, const float *beta, const float *S0,
                       const int32_t *cu_seqlens, int64_t B_or_N, int64_t T,
                       int64_t H, int64_t dk, int64_t dv, void *O, float *S_tok,
                       void *stream) {
    if (!dims_ok(B_or_N) || !dims_ok(T) || H <= 0 || H >= 65536) return GDN_ERR_INVALID_ARG;
    const int64_t N = B_or_N;
    const int64_t rows = cu_seqlens ? T : N * T;
    if (rows > 0 && (!q || !k || !v || !g || !beta || !O || !S_tok)) return GDN_ERR_INVALID_ARG;
    if (io_dtype != GDN_F32 && io_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (dk != gdn::kHeadDim || dv != gdn::kHeadDim) return GDN_ERR_UNSUPPORTED;
    for (const void *p : {q, k, v, static_cast<const void *>(O), static_cast<const void *>(S_tok)})
        if (!aligned(p, 16)) return GDN_ERR_INVALID_ARG;
    if (S0 && !aligned(S0, 16)) return GDN_ERR_INVALID_ARG;
    if (!aligned(g, 4) || !aligned(beta, 4) || (cu_seqlens && !aligned(cu_seqlens, 4)))
        return GDN_ERR_INVALID_ARG;

    if (N * H >= kMaxDim / 2) return GDN_ERR_INVALID_ARG;   // two workgroups per unit
    const int64_t state_elems = gdn::kHeadDim * gdn::kHeadDim;
    if (rows > (int64_t(1) << 44) / (H * state_elems)) return GDN_ERR_INVALID_ARG;
    const int64_t esz = io_dtype == GDN_BF16 ? 2 : 4;
    const int64_t tok_bytes = rows * H * gdn::kHeadDim * esz;
    const int64_t gb_bytes = rows * H * 4;
    const int64_t st_bytes = N * H * state_elems * 4;
    const int64_t stok_bytes = rows * H * state_elems * 4;

    const Range rq = span_of(q, tok_bytes), rk = span_of(k, tok_bytes),
                rv = span_of(v, tok_bytes), rg = span_of(g, gb_bytes),
                rb = span_of(beta, gb_bytes), rO = span_of(O, tok_bytes),
                rSt = span_of(S_tok, stok_bytes),
                rS0 = S0 ? span_of(S0, st_bytes) : Range{0, 0};
    for (Range r : {rq, rk, rv, rg, rb, rS0, rSt})
        if (overlap(rO, r)) return GDN_ERR_ALIAS;
    for (Range r : {rq, rk, rv, rg, rb, rS0})
        if (overlap(rSt, r)) return GDN_ERR_ALIAS;

    gdn::PrefillArgs a{q, k, v, g, beta, S0, cu_seqlens, N, T, H, 0,
                       io_dtype == GDN_BF16, O, nullptr};
    if (N == 0) return GDN_OK;
    if (const int sc = check_seqlens_debug(cu_seqlens, N, T, stream)) return sc;
    hipError_t e = gdn::launch_prefill_states(a, S_tok, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int gdn_preop(const void *xq, const void *xk, const void *xv, int io_dtype, const float *a,
              const float *b, const float *conv_w, const void *state_in, void *state_out,
              const int32_t *cu_seqlens, int64_t B_or_N, int64_t T, int64_t H, int64_t dk,
              int64_t dv, int64_t kernel_size, float eps, void *q, void *k, void *v, float *g,
              float *beta, void *stream) {
    if (!dims_ok(B_or_N) || !dims_ok(T) || H <= 0 || H >= 65536) return GDN_ERR_INVALID_ARG;
    const int64_t N = B_or_N;
    const int64_t rows = cu_seqlens ? T : N * T;
    if (rows > 0 && (!xq || !xk || !xv || !a || !b || !q || !k || !v || !g || !beta))
        return GDN_ERR_INVALID_ARG;
    if (N > 0 && (!conv_w || !state_in || !state_out)) return GDN_ERR_INVALID_ARG;
    if (io_dtype != GDN_F32 && io_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (dk != gdn::kHeadDim || dv != gdn::kHeadDim || kernel_size != 4) return GDN_ERR_UNSUPPORTED;
    if (!(eps >= 0.f && eps <= FLT_MAX)) return GDN_ERR_INVALID_ARG;
    for (const void *p : {xq, xk, xv, static_cast<const void *>(q), static_cast<const void *>(k),
                          static_cast<const void *>(v), static_cast<const void *>(conv_w), state_in,
                          static_cast<const void *>(state_out)})
        if (!aligned(p, 16)) return GDN_ERR_INVALID_ARG;
    for (const void *p : {static_cast<const void *>(a), static_cast<const void *>(b),
                          static_cast<const void *>(g), static_cast<const void *>(beta),
                          static_cast<const void *>(cu_seqlens)})
        if (!aligned(p, 4)) return GDN_ERR_INVALID_ARG;
    if (N >= kMaxDim) return GDN_ERR_INVALID_ARG;
    if (rows > (int64_t(1) << 40) / (H * gdn::kHeadDim)) return GDN_ERR_INVALID_ARG;
    if ((rows + 127) / 128 >= 65536) return GDN_ERR_INVALID_ARG;     // grid.y of the launch
    const int64_t esz = io_dtype == GDN_BF16 ? 2 : 4;
    const int64_t tok = rows * H * gdn::kHeadDim * esz, gb = rows * H * 4;
    const int64_t st = N * 3 * H * 3 * gdn::kHeadDim * esz, wb = 3 * H * gdn::kHeadDim * 4 * 4;
    const Range rxq = span_of(xq, tok), rxk = span_of(xk, tok), rxv = span_of(xv, tok),
                ra = span_of(a, gb), rb = span_of(b, gb), rw = span_of(conv_w, wb),
                rsi = span_of(state_in, st), rso = span_of(state_out, st),
                rq = span_of(q, tok), rk = span_of(k, tok), rv = span_of(v, tok),
                rg = span_of(g, gb), rbe = span_of(beta, gb);
    for (Range o : {rq, rk, rv, rg, rbe, rso}) {
        for (Range i : {rxq, rxk, rxv, ra, rb, rw})
            if (overlap(o, i)) return GDN_ERR_ALIAS;
    }
    const Range outs[] = {rq, rk, rv, rg, rbe, rso};
    for (int i = 0; i < 6; ++i)
        for (int j = i + 1; j < 6; ++j)
            if (overlap(outs[i], outs[j])) return GDN_ERR_ALIAS;
    for (Range o : {rq, rk, rv, rg, rbe})
        if (overlap(o, rsi)) return GDN_ERR_ALIAS;
    if (overlap(rso, rsi) && rso.lo != rsi.lo) return GDN_ERR_ALIAS;   // in place or apart
    if (N == 0) return GDN_OK;
    if (const int sc = check_seqlens_debug(cu_seqlens, N, T, stream)) return sc;
    gdn::PreopArgs p{xq, xk, xv, a, b, conv_w, state_in, state_out, cu_seqlens, N, T, rows, H,
                     eps, io_dtype == GDN_BF16, q, k, v, g, beta};
    const hipError_t e = gdn::launch_preop(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int gdn_chunk_prefill_preop(const void *xq, const void *xk, const void *xv, int io_dtype,
                            const float *a, const float *b, const float *conv_w,
                            const void *state_in, void *state_out, float eps, const float *S0,
                            const int32_t *cu_seqlens, int64_t B_or_N, int64_t T, int64_t H,
                            int64_t dk, int64_t dv, int64_t kernel_size, int64_t chunk, void *O,
                            float *S_T, void *stream) {
    gdn::PrefillArgs pa{};
    int64_t tok_bytes = 0;
    const int st = check_prefill(xq, xk, xv, io_dtype, a, b, S0, cu_seqlens, B_or_N, T, H, dk,
                                 dv, chunk, O, S_T, pa, tok_bytes);
    if (st != GDN_OK) return st;
    if (io_dtype != GDN_BF16 || chunk != 64 || kernel_size != 4) return GDN_ERR_UNSUPPORTED;
    const int64_t N = B_or_N;
    if (N > 0 && (!conv_w || !state_in || !state_out)) return GDN_ERR_INVALID_ARG;
    if (!(eps >= 0.f && eps <= FLT_MAX)) return GDN_ERR_INVALID_ARG;
    for (const void *p : {static_cast<const void *>(conv_w), state_in,
                          static_cast<const void *>(state_out)})
        if (!aligned(p, 16)) return GDN_ERR_INVALID_ARG;
    const int64_t rows = cu_seqlens ? T : N * T;
    const int64_t gb = rows * H * 4, fifo = N * 3 * H * 3 * gdn::kHeadDim * 2,
                  wb = 3 * H * gdn::kHeadDim * 4 * 4,
                  sb = N * H * gdn::kHeadDim * gdn::kHeadDim * 4;
    const Range rxq = span_of(xq, tok_bytes), rxk = span_of(xk, tok_bytes),
                rxv = span_of(xv, tok_bytes), ra = span_of(a, gb), rb = span_of(b, gb),
                rw = span_of(conv_w, wb), rsi = span_of(state_in, fifo),
                rso = span_of(state_out, fifo), rO = span_of(O, tok_bytes),
                rST = span_of(S_T, sb), rS0 = S0 ? span_of(S0, sb) : Range{0, 0};
    // the FIFO out is exactly the FIFO in, or apart from every other buffer
    for (Range r : {rxq, rxk, rxv, ra, rb, rw, rO, rST, rS0})
        if (overlap(rso, r)) return GDN_ERR_ALIAS;
    if (overlap(rso, rsi) && rso.lo != rsi.lo) return GDN_ERR_ALIAS;
    // the outputs O and S_T are apart from the weights and the FIFO in
    for (Range r : {rw, rsi})
        if (overlap(rO, r) || overlap(rST, r)) return GDN_ERR_ALIAS;
    if (N == 0) return GDN_OK;
    if (const int sc = check_seqlens_debug(cu_seqlens, N, T, stream)) return sc;
    pa.conv_w = conv_w;
    pa.fifo = state_in;
    pa.ceps = eps;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (gdn::launch_prefill_mfma(pa, s) != hipSuccess) return GDN_ERR_HIP;
    // the FIFO update after the prompt kernel, which read state_in
    gdn::PreopArgs p{xq, xk, xv, a, b, conv_w, state_in, state_out, cu_seqlens, N, T, rows, H,
                     eps, true, nullptr, nullptr, nullptr, nullptr, nullptr};
    return gdn::launch_preop_state(p, s) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

namespace {
int decode_step(const void *q, const void *k, const void *v, int io_dtype, const float *g,
                const float *beta, float *S, int64_t B, int64_t H, int64_t dk, int64_t dv,
                void *o, bool stream_state, void *stream) {
    if (!q || !k || !v || !g || !beta || !S || !o) return GDN_ERR_INVALID_ARG;
    if (!dims_ok(B) || H <= 0 || H >= 65536) return GDN_ERR_INVALID_ARG;
    if (io_dtype != GDN_F32 && io_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (dk != gdn::kHeadDim || dv != gdn::kHeadDim) return GDN_ERR_UNSUPPORTED;
    for (const void *p : {q, k, v, static_cast<const void *>(o), static_cast<const void *>(S)})
        if (!aligned(p, 16)) return GDN_ERR_INVALID_ARG;
    if (!aligned(g, 4) || !aligned(beta, 4)) return GDN_ERR_INVALID_ARG;
    const int64_t units = B * H;
    if (units >= kMaxDim / 2) return GDN_ERR_INVALID_ARG;   // two workgroups per head
    const int64_t esz = io_dtype == GDN_BF16 ? 2 : 4;
    const int64_t vec_bytes = units * gdn::kHeadDim * esz;
    const Range rq = span_of(q, vec_bytes), rk = span_of(k, vec_bytes),
                rv = span_of(v, vec_bytes), rg = span_of(g, units * 4),
                rb = span_of(beta, units * 4), ro = span_of(o, vec_bytes),
                rS = span_of(S, units * gdn::kHeadDim * gdn::kHeadDim * 4);
    for (Range r : {rq, rk, rv, rg, rb, rS})
        if (overlap(ro, r)) return GDN_ERR_ALIAS;
    for (Range r : {rq, rk, rv, rg, rb})
        if (overlap(rS, r)) return GDN_ERR_ALIAS;
    if (units == 0) return GDN_OK;
    gdn::DecodeArgs a{q, k, v, g, beta, S, units, io_dtype == GDN_BF16, o};
    a.stream_state = stream_state;
    hipError_t e = gdn::launch_decode(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}
}  // namespace

int gdn_decode_step(const void *q, const void *k, const void *v, int io_dtype,
                    const float *g, const float *beta, float *S, int64_t B,
                    int64_t H, int64_t dk, int64_t dv, void *o, void *stream) {
    return decode_step(q, k, v, io_dtype, g, beta, S, B, H, dk, dv, o, false, stream);
}

int gdn_decode_step_preop(const void *xq, const void *xk, const void *xv, int io_dtype,
                          const float *a, const float *b, const float *conv_w,
                          const void *state_in, void *state_out, float eps, const void *z,
                          const float *norm_w, float norm_eps, float *S, int64_t B, int64_t H,
                          int64_t dk, int64_t dv, int state_hint, void *o, void *stream) {
    if (state_hint != GDN_STATE_CACHED && state_hint != GDN_STATE_STREAMING)
        return GDN_ERR_UNSUPPORTED;
    if (!xq || !xk || !xv || !a || !b || !conv_w || !state_in || !state_out || !S || !o)
        return GDN_ERR_INVALID_ARG;
    if (!dims_ok(B) || H <= 0 || H >= 65536) return GDN_ERR_INVALID_ARG;
    if (io_dtype != GDN_F32 && io_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (dk != gdn::kHeadDim || dv != gdn::kHeadDim) return GDN_ERR_UNSUPPORTED;
    if (!(eps >= 0.f && eps <= FLT_MAX)) return GDN_ERR_INVALID_ARG;
    if (z && (!norm_w || !aligned(z, 16) || !aligned(norm_w, 4) ||
              !(norm_eps >= 0.f && norm_eps <= FLT_MAX)))
        return GDN_ERR_INVALID_ARG;
    for (const void *p : {xq, xk, xv, static_cast<const void *>(conv_w), state_in,
                          static_cast<const void *>(state_out), static_cast<const void *>(S),
                          static_cast<const void *>(o)})
        if (!aligned(p, 16)) return GDN_ERR_INVALID_ARG;
    if (!aligned(a, 4) || !aligned(b, 4)) return GDN_ERR_INVALID_ARG;
    const int64_t units = B * H;
    if (units >= kMaxDim) return GDN_ERR_INVALID_ARG;
    const int64_t esz = io_dtype == GDN_BF16 ? 2 : 4;
    const int64_t vec = units * gdn::kHeadDim * esz, gbytes = units * 4;
    const int64_t fifo = units * 3 * 3 * gdn::kHeadDim * esz;
    const Range rxq = span_of(xq, vec), rxk = span_of(xk, vec), rxv = span_of(xv, vec),
                ra = span_of(a, gbytes), rb = span_of(b, gbytes),
                rw = span_of(conv_w, 3 * H * gdn::kHeadDim * 4 * 4),
                rsi = span_of(state_in, fifo), rso = span_of(state_out, fifo),
                rS = span_of(S, units * gdn::kHeadDim * gdn::kHeadDim * 4), ro = span_of(o, vec);
    // outputs (o, S, the new FIFO) apart from every input and from each other;
    // the FIFO may be advanced in place
    const Range rz = z ? span_of(z, vec) : Range{0, 0},
                rnw = z ? span_of(norm_w, gdn::kHeadDim * 4) : Range{0, 0};
    for (Range out : {ro, rS, rso})
        for (Range in : {rxq, rxk, rxv, ra, rb, rw, rz, rnw})
            if (overlap(out, in)) return GDN_ERR_ALIAS;
    if (overlap(ro, rS) || overlap(ro, rso) || overlap(rS, rso)) return GDN_ERR_ALIAS;
    if (overlap(ro, rsi) || overlap(rS, rsi)) return GDN_ERR_ALIAS;
    if (overlap(rso, rsi) && rso.lo != rsi.lo) return GDN_ERR_ALIAS;
    if (units == 0) return GDN_OK;
    gdn::DecodePreopArgs p{xq, xk, xv, a, b, conv_w, state_in, state_out, eps, S, units, H,
                           io_dtype == GDN_BF16, o, state_hint == GDN_STATE_STREAMING};
    p.z = z;
    p.norm_w = norm_w;
    p.norm_eps = norm_eps;
    const hipError_t e = gdn::launch_decode_preop(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int gdn_decode_step_ex(const void *q, const void *k, const void *v, int io_dtype,
                       const float *g, const float *beta, float *S, int64_t B,
                       int64_t H, int64_t dk, int64_t dv, int state_hint, void *o,
                       void *stream) {
    if (state_hint != GDN_STATE_CACHED && state_hint != GDN_STATE_STREAMING)
        return GDN_ERR_UNSUPPORTED;
    return decode_step(q, k, v, io_dtype, g, beta, S, B, H, dk, dv, o,
                       state_hint == GDN_STATE_STREAMING, stream);
}

}  // extern "C"
