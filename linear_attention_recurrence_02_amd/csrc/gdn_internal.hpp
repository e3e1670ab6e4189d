// Internal declarations shared by the translation units of libgdn (not part of
// the public ABI; see include/gdn.h for that).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <cstdint>

namespace gdn {

constexpr int kHeadDim = 128;   // dk == dv == 128: the page's per-head state size

constexpr int kInverseDefault = 0;        // the kernel's own choice
constexpr int kInverseSubstitution = 1;   // back substitution on the vector ALUs
constexpr int kInverseDoubling = 2;       // block doubling on the matrix cores

constexpr int kColumnsDefault = 0;        // the launch's own choice
constexpr int kColumnsWhole = 1;          // one workgroup per (sequence, head)
constexpr int kColumnsSplit = 2;          // two, of 64 value columns each

// A validated prompt-form call.  Token rows are counted in units of H heads:
// the element (row r, head h, dim i) of q/k/v/O sits at ((r * H) + h) * 128 + i.
struct PrefillArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    const float *S0;            // may be null (zero state)
    const int32_t *cu_seqlens;  // may be null (uniform batch)
    int64_t N;                  // sequences
    int64_t T;                  // tokens per sequence (uniform) or total (packed)
    int64_t H;                  // heads
    int chunk;                  // 16, 32 or 64
    bool bf16;                  // io dtype of q/k/v (and of O unless out_f32)
    void *O;
    float *S_T;
    // bf16 inputs with an fp32 O (the matrix-core kernels' arithmetic without
    // the rounding of O to bf16).
    bool out_f32 = false;
    // Gated RMS norm on the output rows (null z: plain O).  O then receives
    // y = norm_w * O / sqrt(mean(O^2) + eps) * silu(z), z with the io dtype.
    const void *z = nullptr;
    const float *norm_w = nullptr;
    float eps = 0.f;
    // How the matrix-core kernel forms the diagonal 16 x 16 blocks of
    // (I + N)^-1 (the vector kernel always substitutes column by column).
    int inverse = kInverseDefault;
    // Whether the matrix-core kernel splits each unit's value columns over two
    // workgroups (the other kernels ignore it).
    int columns = kColumnsDefault;
    // Whether a batch of short sequences may take the 16-token kernel (off
    // when the caller names the matrix-core kernel's inverse method).
    bool short_ok = true;
    // The pre-operations fused into the 64-token kernel's chunk load (non-null
    // conv_w): q, k, v, g, beta are then the raw projections xq, xk, xv and the
    // gate inputs a, b; fifo is the conv FIFO state [N, 3, H, 3, 128] (bf16)
    // read for the rows before each sequence, and ceps the norm's eps.
    const float *conv_w = nullptr;
    const void *fifo = nullptr;
    float ceps = 0.f;
};

struct DecodeArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    float *S;
    int64_t units;              // B * H
    bool bf16;
    void *o;
    // Non-temporal state loads and stores: for states that are not in cache
    // anyway (many layers or batches in turn), at the cost of the cache
    // benefit when one small batch is stepped over and over.
    bool stream_state = false;
};

// A validated decode step with the pre-operations fused in front.
struct DecodePreopArgs {
    const void *xq, *xk, *xv;   // raw projections [units, 128]
    const float *a, *b;         // gate inputs [units]
    const float *conv_w;        // [3, H, 128, 4]
    const void *state_in;       // FIFO [N, 3, H, 3, 128] io dtype
    void *state_out;            // same shape: exactly state_in, or disjoint
    float eps;
    float *S;                   // [units, 128, 128]
    int64_t units, H;
    bool bf16;
    void *o;
    bool stream_state;
    // Gated RMS norm on the output row (null z: plain o)
    const void *z = nullptr;
    const float *norm_w = nullptr;
    float norm_eps = 0.f;
};

// A validated pre-operation call (conv FIFO, silu, L2 norm, gates).
struct PreopArgs {
    const void *xq, *xk, *xv;   // raw projections [rows, H, 128]
    const float *a, *b;         // gate inputs [rows, H]
    const float *conv_w;        // [3, H, 128, 4]
    const void *state_in;       // [N, 3, H, 3, 128], io dtype
    void *state_out;            // same shape; may be state_in
    const int32_t *cu_seqlens;  // may be null
    int64_t N, T, rows, H;
    float eps;
    bool bf16;
    void *q, *k, *v;
    float *g, *beta;
};

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_decode_preop(const DecodePreopArgs &a, hipStream_t stream);
// Helpers of the segmented prompt form (see gdn_segmented.hip).
hipError_t launch_segment_prep(const int32_t *cu_in, int64_t N, int64_t T, int64_t L, int64_t Ns,
                               int32_t *seg, int32_t *cu_out, float *sid, int64_t units,
                               hipStream_t stream);
hipError_t launch_segment_scan(const float *M, const float *B, const float *S0, float *Sin,
                               const int32_t *seg, int64_t N, int64_t H, hipStream_t stream);
hipError_t launch_segment_gather(const float *Sout, const float *S0, const int32_t *seg,
                                 float *S_T, int64_t N, int64_t H, hipStream_t stream);
hipError_t launch_preop(const PreopArgs &p, hipStream_t stream);
// The FIFO update of a pre-operation call alone (state_out from state_in and
// the raw rows), after every read of state_in on the same stream.
hipError_t launch_preop_state(const PreopArgs &p, hipStream_t stream);
hipError_t launch_prefill_valu(const PrefillArgs &a, hipStream_t stream);
hipError_t launch_prefill_mfma(const PrefillArgs &a, hipStream_t stream);
bool prefill_mfma_supports(const PrefillArgs &a);
hipError_t launch_prefill_short(const PrefillArgs &a, hipStream_t stream);
bool prefill_short_pays(const PrefillArgs &a);
// The prompt form keeping the state after every token in S_tok (chunk unused).
hipError_t launch_prefill_states(const PrefillArgs &a, float *S_tok, hipStream_t stream);
// Compute units of the current device, 0 if they cannot be queried (cached
// per device; launch heuristics use it).
int compute_units();

// ---- small device helpers -------------------------------------------------

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__hip_bfloat16 x) { return __bfloat162float(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __hip_bfloat16 from_f32<__hip_bfloat16>(float x) {
    return __float2bfloat16(x);   // round to nearest even
}

// Packed batches of at most this many sequences are walked longest first.
constexpr int64_t kMaxRankedSequences = 1024;

// The sequence a workgroup of a packed batch takes so that the longest
// sequences start first: the one of rank p when sequences are ordered by
// length, longest first, ties by index (a permutation of 0..N-1).  Every
// thread of the workgroup calls it with the same lens buffer (LDS, room for
// kMaxRankedSequences + 3 ints): the lengths, from the clamped offsets as
// everywhere else, are staged there once, then each thread ranks a share of
// the sequences by counting, and the one whose rank is p is left in *slot.
// The caller synchronises the workgroup before reading *slot.
__device__ __forceinline__ void rank_longest_first(const int32_t *cu, int64_t N, int64_t T,
                                                   int64_t p, int tid, int nthreads,
                                                   int32_t *lens, int64_t *slot) {
    const int n4 = static_cast<int>((N + 3) / 4) * 4;
    for (int n = tid; n < n4; n += nthreads) {
        int32_t l = -1;                              // padding ranks below every sequence
        if (n < N) {
            int64_t a = cu[n], b = cu[n + 1];
            a = a < 0 ? 0 : (a > T ? T : a);
            b = b < a ? a : (b > T ? T : b);
            l = static_cast<int32_t>(b - a);
        }
        lens[n] = l;
    }
    __syncthreads();
    for (int n = tid; n < N; n += nthreads) {
        const int32_t ln = lens[n];
        int rank = 0;
        for (int m = 0; m < n4; m += 4) {
            const int4 l4 = *reinterpret_cast<const int4 *>(&lens[m]);
            rank += (l4.x > ln) || (l4.x == ln && m < n);
            rank += (l4.y > ln) || (l4.y == ln && m + 1 < n);
            rank += (l4.z > ln) || (l4.z == ln && m + 2 < n);
            rank += (l4.w > ln) || (l4.w == ln && m + 3 < n);
        }
        if (rank == p) *slot = n;
    }
}

// Sequence span of unit n: first token row and length.  Offsets from the
// device are clamped into [0, T] so that a malformed array cannot make a
// kernel read or write outside the caller's buffers.
__device__ __forceinline__ void sequence_span(const int32_t *cu, int64_t n, int64_t T,
                                              int64_t &start, int64_t &len) {
    if (cu) {
        int64_t a = cu[n], b = cu[n + 1];
        a = a < 0 ? 0 : (a > T ? T : a);
        b = b < a ? a : (b > T ? T : b);
        start = a;
        len = b - a;
    } else {
        start = n * T;
        len = T;
    }
}

}  // namespace gdn
