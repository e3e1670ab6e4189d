// Chunkwise-parallel prompt form on the gfx950 matrix cores (bf16 inputs,
// 64-token chunks, fp32 state and accumulation, fp16 and bf16 matrix operands,
// split into hi + lo pairs where the recurrence needs it).
//
// The form (Qwen3.5-9B-npu model page, "How it works" -> "Gated DeltaNet on
// the NPU"), per chunk of C = 64 tokens with incoming state S (dk x dv):
//     G  = cumsum(g)                                    inclusive, in the chunk
//     N  = diag(beta) [exp(G_t - G_j) k_t.k_j]_{j<t}     strictly lower
//     D  = (I + N)^-1 diag(beta) (V - diag(exp G) K S)   per-token deltas
//     O  = diag(exp G) Q S + A D,  A = [exp(G_t - G_j) q_t.k_j]_{j<=t}
//     S <- exp(G_C) S + K^T diag(exp(G_C - G)) D
// Rows past a sequence's end are the page's token_valid padding (g = 0,
// beta = 0, zero q/k/v): they leave S untouched and are not stored.
//
// Only three products touch S, so everything else is prepared off the serial
// path.  With T = (I + N)^-1 the deltas split as D = U - W S, where
//     W = T diag(beta exp G) K,   U = T diag(beta) V
// depend on the chunk alone.  W and U are found without forming T: on the four
// 16-token blocks i of the chunk, with T_ii = (I + N_ii)^-1,
//     W_i = P_i K_i - sum_{j<i} M_ij W_j,   P_i = T_ii diag(beta exp G)_i,
//     U_i = P'_i V_i - sum_{j<i} M_ij U_j,  P'_i = T_ii diag(beta)_i,
//     M_ij = T_ii N_ij,
// which is block forward substitution on (I + N) W = diag(beta exp G) K.
//
// One 512-thread workgroup (8 waves) per (sequence, head), two roles:
//   * consumer waves 0..3 walk the chunks in order.  Wave w owns dv columns
//     [32w, 32w+32) of S, D, U and O; its share of S lives in 8 x 2 result
//     tiles of v_mfma_f32_16x16x32_f16 (16 dk rows x 16 dv columns, 4 fp32 per
//     lane: lane l holds rows 4(l/16)..+3 of column l%16) for the whole walk.
//     Per chunk: D = U - W S, S <- exp(G_C) S + K^T diag(exp(G_C - G)) D,
//     O = diag(exp G) Q S + A D with the S that entered the chunk, and the W/U
//     block substitution of the next chunk (its own 32 columns of W and U; U
//     stays in registers).  S and D enter the products straight from their
//     result tiles: a result tile is the B operand of a product over its rows
//     when the partner A operand is read in the matching k order (lane group q
//     takes k = 4q..4q+3 and 16+4q..16+4q+3 of a 32-wide k step), and, read
//     as an A operand, it is its own transpose (O is computed as O^T).  K^T,
//     V and W are read with the gfx950 LDS transpose load, which turns four
//     16-element rows into one column per lane.
//   * producer waves 4..7 prepare chunk c+1 while the consumers work on chunk
//     c: the Gram tiles K K^T and K Q^T (exact products of fp16 copies of the
//     bf16 inputs, fp32 accumulation) with the decay and beta applied on the
//     accumulators; T_ii (one block per wave) by the page's exact block
//     doubling on the matrix cores (or, selectable, by fp32 back
//     substitution) and M_ij = T_ii N_ij; and the staging of chunk c+2 (rows
//     prefetched into registers a period earlier; K and Q converted to fp16,
//     V kept as bf16).
//   Each chunk period has three barrier-separated phases:
//     1: consumers D, state update (chunk c)  | producers store V (c+1), then
//                                            |   load V (c+2); Gram tiles (c+1)
//     2: consumers O (chunk c)               | producers T_ii, P_i, M_ij (c+1)
//     3: consumers W, U (chunk c+1)          | producers store A (c+1); convert
//                                            |   c+2's K and Q, store them and
//                                            |   the scalars; each stream's
//                                            |   loads for c+3 go out as soon
//                                            |   as its registers are free
//   Each array is written in a phase in which nobody reads it: K, Q and the
//   per-token scalars are double-buffered, everything else is single.
//   The two roles run as two separate loops under a wave-uniform branch and
//   execute the same number of barriers (1 + 3 (nch + 1)).  The consumers'
//   work sets phases 1 to 3 of the plain form; with the pre-operations fused
//   in, the producers set phases 2 and 3 and take wave priority in them.
// A null v stands for zero values and a null O for no output rows (the
// segmented form's state-map runs).
// Template variants: kGated fuses the block's gated RMS norm into the output
// step (each consumer wave loads its gate rows into registers at the start of
// phase 2; the four consumer waves exchange per-row sums of O^2 through LDS);
// kDoubling picks the T_ii method; kRank
// walks a packed batch longest first (each workgroup ranks the sequence
// lengths before the roles split, one barrier that both roles execute);
// kPreop runs the block's pre-operations (causal conv over the FIFO window,
// silu, L2 norm of q and k, g = -softplus(a), beta = sigmoid(b); the
// Qwen3.5-4B -- Hexagon NPU (QHexRT) -- v81 page's text decoder description
// and the QCS6490 page's port notes) in the producers' staging step, from the
// raw projections: each producer lane holds two channels of its block's rows
// and of the three rows before them, so the conv window stays in the lane; K's
// pre-operations run in phase 2 after the inverse chain, q's and v's in
// phase 3 beside the consumers' W/U step; NCC = 1 splits the value columns of
// each (sequence, head) over two workgroups of 64 columns (consumer waves of
// 16 columns each, the producers' work and W repeated in both), for launches
// whose workgroups then still all fit on the CUs at once.
// Precision.  The state, the accumulators, U and the per-token scalars are
// fp32.  K and Q enter the products as fp16 copies of the bf16 inputs, V as
// the bf16 input itself (in bf16 products against P').  Correlated keys (the
// page's own warning about real keys in reduced precision) make the chunk's
// deltas large next to what is built from them: the terms of A D and of
// K^T D nearly cancel, and so do those of the U chain.  An operand rounded
// once to fp16 (2^-11) is not enough there, so A, D, the decayed D, P, P',
// N_ij, M_ij, T_ii inside the doubling and the U chain enter their products
// as hi + lo pairs (fp16, about 2^-22; P' as a bf16 pair against the bf16 V),
// while S and W, whose single rounding is harmless, stay single fp16
// operands.  Each consumer wave holds its value-side quantities (its state
// columns and everything linear in them: U, D, O) at a power-of-two scale
// chosen per chunk so that their largest entry lies in [8, 16), which keeps
// fp16's relative precision for heads of any magnitude (the page's small
// heads, 1e-3..2e-2, and far smaller or larger ones); the scale is exact and
// is removed when O and S_T are stored.

#include "gdn_mfma.hpp"

namespace gdn {
namespace {

constexpr int C = 64;             // chunk length
constexpr int D = kHeadDim;       // 128
constexpr int KS = D + 16;        // fp16 row stride of the token-major K and V tiles
constexpr int QS = D + 12;        // fp16 row stride of the token-major Q tiles
constexpr int WS = C + 16;        // fp16 row stride of W (dk-major)
constexpr int AS = C + 4;         // fp16 row stride of A (token-major)
constexpr int BS = 16 + 8;        // fp16 row stride of the 16 x 16 blocks T_ii, P_i, P'_i, M_ij
constexpr int NS = 20;            // fp32 row stride of the diagonal blocks of N
// How the diagonal blocks of (I + N)^-1 are formed unless the caller names a
// method: block doubling on the matrix cores (true) or fp32 back substitution.
// Doubling measured 2-6% faster at every launch size from 4 to 512 units of
// 4096 tokens (its producers also keep their lane masks out of the chunk loop).
constexpr bool kDefaultDoubling = true;

// LDS layouts.  Each array's row stride (and, for K, V and W, an XOR of the
// column with a few row bits) is chosen so that its main access patterns hit
// 32 distinct banks per 128-byte wavefront slice: the 16-byte row reads and the
// four-row transpose loads of K and V, the 8-byte row reads of Q and A, and the
// transpose loads and 8-byte writes of W.  Every swizzle term is a per-lane
// constant, so each address is a per-lane base plus a compile-time offset.
struct __attribute__((aligned(16))) Smem {
    f16 K[2][C * KS];             // keys, double-buffered; column c of row t at c ^ ksw(t)
    bf16 V[C * KS];               // values (the bf16 inputs as they are), same layout as K
    f16 Q[2][C * QS];             // queries, double-buffered
    f16 W[D * WS];                // -W, dk-major: -W_td at d * WS + (t ^ wsw(d))
    f16 A[2][C * AS];             // decayed masked Q K^T, token-major: hi, lo
    float NR[4][16 * NS];         // diagonal blocks of N, row-major
    f16 P[2][4][16 * BS];         // T_ii diag(beta exp G): hi, lo
    bf16 Pv[2][4][16 * BS];       // T_ii diag(beta): hi, lo (bf16, against the bf16 V)
    f16 M[2][6][16 * BS];         // -T_ii N_ij, i > j: hi, lo
    float G2[2][C];               // cumsum(g) * log2(e)
    float EG[2][C];               // exp(G_t)
    float EC[2][C];               // exp(G_last - G_t)
    float Bt[2][C];               // beta
    float NP[C][4];               // gated norm: per-wave partial sums of O^2 by token row
    float NW[D];                  // gated norm: weights
    uint32_t NPC;                 // gated norm: partial-sum sets posted by consumer waves
};

// Column swizzles: K and V flip column bit 3 with row bit 2; W flips column
// bits 2..3 with row bits 2..3.
__device__ __forceinline__ int ksw(int row) { return ((row >> 2) & 1) << 3; }
__device__ __forceinline__ int wsw(int row) { return ((row >> 2) & 3) << 2; }

// index of the off-diagonal block (i, j), i > j, in Smem::M
__device__ __forceinline__ constexpr int oblk(int i, int j) { return i * (i - 1) / 2 + j; }

// Loads are always issued, rows past the chunk reading the sequence's first row
// instead, so that every period issues the same load sequence; the tail mask is
// applied when the rows are staged.
__device__ __forceinline__ void load_rows(f32x4 *dst, const bf16 *src, int64_t start, int64_t row0,
                                          int r, int nv, int64_t H, int64_t h, int q) {
    const bf16 *p = src + ((r < nv ? row0 + r : start) * H + h) * D + 8 * q;
#pragma unroll
    for (int s = 0; s < 4; ++s) dst[s] = *reinterpret_cast<const f32x4 *>(p + 32 * s);
}
// Rows of one 16-token block held by a producer lane (row r, columns
// 32s + 8q..+7 for s = 0..3), converted in place from bf16 to fp16; rows at or
// past nv are zeroed (only a sequence's last chunk has such rows).
__device__ __forceinline__ void to_fp16_rows(f32x4 *x, int r, int nv) {
#pragma unroll
    for (int s = 0; s < 4; ++s) x[s] = __builtin_bit_cast(f32x4, bf_to_h8(x[s]));
    if (nv < C) {
        const bool ok = r < nv;
#pragma unroll
        for (int s = 0; s < 4; ++s) x[s] = ok ? x[s] : zero4();
    }
}
// The same rows kept as bf16 (V): only the tail rows are zeroed.
__device__ __forceinline__ void mask_rows(f32x4 *x, int r, int nv) {
    if (nv < C) {
        const bool ok = r < nv;
#pragma unroll
        for (int s = 0; s < 4; ++s) x[s] = ok ? x[s] : zero4();
    }
}
__device__ __forceinline__ void store_rows_kv(void *tile_, const f32x4 *x, int r, int q) {
    f16 *tile = static_cast<f16 *>(tile_);
    const int c = (8 * q) ^ ksw(r);
#pragma unroll
    for (int s = 0; s < 4; ++s) *reinterpret_cast<f32x4 *>(&tile[r * KS + 32 * s + c]) = x[s];
}
// Q rows are only 8-byte aligned (QS is 2 mod 4 words): two 8-byte stores.
__device__ __forceinline__ void store_rows_q(f16 *tile, const f32x4 *x, int r, int q) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        f32x2 *d = reinterpret_cast<f32x2 *>(&tile[r * QS + 32 * s + 8 * q]);
        d[0] = f32x2{x[s][0], x[s][1]};
        d[1] = f32x2{x[s][2], x[s][3]};
    }
}

// A DPP move within rows of 16 lanes (every lane has a source for the
// controls used here).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Sums over the 64 lanes of a wave of 16 values per lane (x[r] for block row
// r), by halving exchanges: at each step a lane keeps the rows of one half,
// adds its partner's values of those rows and hands over the other half in
// exchange.  Lane bits 5, 4, 3 and 2 pick the halves (partners l ^ 32, l ^ 16,
// l ^ 8, then l ^ 7 within each eight lanes), and the last two steps add the
// four lanes of a quad, so lane l returns the sum of row
// 8 (l >> 5 & 1) + 4 (l >> 4 & 1) + 2 (l >> 3 & 1) + (l >> 2 & 1).
__device__ __forceinline__ float rows16_wave_sum(const float *x, int l) {
    const bool b5 = (l >> 5) & 1, b4 = (l >> 4) & 1, b3 = (l >> 3) & 1, b2 = (l >> 2) & 1;
    float y[8], z[4], w[2];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        y[i] = (b5 ? x[i + 8] : x[i]) + __shfl_xor(b5 ? x[i] : x[i + 8], 32);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        z[i] = (b4 ? y[i + 4] : y[i]) + __shfl_xor(b4 ? y[i] : y[i + 4], 16);
#pragma unroll
    for (int i = 0; i < 2; ++i)
        w[i] = (b3 ? z[i + 2] : z[i]) + dpp_mov<0x128>(b3 ? z[i] : z[i + 2]);   // row_ror:8
    float t = (b2 ? w[1] : w[0]) + dpp_mov<0x141>(b2 ? w[0] : w[1]);         // row_half_mirror
    t += dpp_mov<0xb1>(t);                                                    // quad_perm [1,0,3,2]
    t += dpp_mov<0x4e>(t);                                                    // quad_perm [2,3,0,1]
    return t;
}

struct Unit {
    const bf16 *q, *k, *v;
    const float *g, *beta;
    int64_t start, len, H, h;
    // fused pre-operations: q, k, v, g, beta are then the raw projections and
    // gate inputs; the conv FIFO state of the sequence and the conv weights
    const bf16 *fifo;
    const float *conv_w;
    int64_t seq;
    float ceps;
    __device__ int rows_in(int pc) const {
        const int64_t rem = len - int64_t(pc) * C;
        return static_cast<int>(rem < 0 ? 0 : (rem < C ? rem : C));
    }
    __device__ int64_t row0(int pc) const { return start + int64_t(pc) * C; }
};

// Producer wave p = 4..7 - 4 (lane r16 + 16 q) stages rows 16p + r16 of each
// chunk from registers loaded a period ahead.  K and Q (and token l's g and
// beta, for wave p = 0, which scans them) of chunk c+2 are converted and
// stored in phase 3 of period c, into the buffers the consumers' W/U step does
// not read, and each stream's loads for chunk c+3 go out as soon as its
// registers are free.  V is single-buffered (the W/U step of phase 3 reads
// it): V of chunk c+1 is stored in phase 1 of period c, and the loads of V of
// chunk c+2 follow at once into the same registers.
struct Producer {
    f32x4 pK[4], pV[4], pQ[4];
    float pg, pb;
    float sg2, seg, sec, sbt;     // scan results of the staged chunk (wave p = 0)
    h4x2 Ah[4];                   // A tiles of the chunk being prepared, hi/lo (phase 1 -> 3)
    h4x2 Nop[3];                  // off-diagonal N blocks of the chunk, hi/lo (phase 1 -> 2)

    __device__ void load_v(const Unit &u, int pc, int p, int r16, int q) {
        if (u.v) {
            load_rows(pV, u.v, u.start, u.row0(pc), 16 * p + r16, u.rows_in(pc), u.H, u.h, q);
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) pV[s] = zero4();
        }
    }
    __device__ void load_k(const Unit &u, int pc, int p, int r16, int q) {
        load_rows(pK, u.k, u.start, u.row0(pc), 16 * p + r16, u.rows_in(pc), u.H, u.h, q);
    }
    __device__ void load_q(const Unit &u, int pc, int p, int r16, int q) {
        load_rows(pQ, u.q, u.start, u.row0(pc), 16 * p + r16, u.rows_in(pc), u.H, u.h, q);
    }
    __device__ void load_gates(const Unit &u, int pc, int l) {
        const int64_t gi = (l < u.rows_in(pc) ? u.row0(pc) + l : u.start) * u.H + u.h;
        pg = u.g[gi];
        pb = u.beta[gi];
    }
    // Phase 3: K and Q of the chunk in the registers (nv rows) converted to
    // fp16 (rows past nv zeroed) and stored in buffer set nb, with the
    // per-token scalars (wave p = 0); each stream's registers then take the
    // loads of chunk pn.
    __device__ void stage_kq(Smem &sm, int nb, int nv, int p, int l, int r16, int q, const Unit &u, int pn) {
        to_fp16_rows(pK, 16 * p + r16, nv);
        store_rows_kv(sm.K[nb], pK, 16 * p + r16, q);
        load_k(u, pn, p, r16, q);
        to_fp16_rows(pQ, 16 * p + r16, nv);
        store_rows_q(sm.Q[nb], pQ, 16 * p + r16, q);
        load_q(u, pn, p, r16, q);
        if (p == 0) {
            scan(nv, l);
            store_scalars(sm, nb, p, l);
            load_gates(u, pn, l);
        }
    }
    // Phase 1: V of the chunk in the registers (nv rows, the rest zeroed) to
    // LDS, then the loads of chunk pn.
    __device__ void stage_v(Smem &sm, int nv, int p, int r16, int q, const Unit &u, int pn) {
        mask_rows(pV, 16 * p + r16, nv);
        store_rows_kv(sm.V, pV, 16 * p + r16, q);
        load_v(u, pn, p, r16, q);
    }
    // The per-token scalars of the staged chunk from g and beta (wave p = 0,
    // lane l = token l; rows past nv take g = 0, beta = 0).
    __device__ void scan(int nv, int l) {
        const bool okl = l < nv;
        sbt = okl ? pb : 0.f;
        sg2 = log2e_times(wave_prefix_sum(okl ? bounded_log_decay(pg) : 0.f));
        const float last = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sg2), 63));
        seg = __builtin_amdgcn_exp2f(sg2);
        sec = __builtin_amdgcn_exp2f(last - sg2);
    }

    // ---- staging with the pre-operations fused in (kPreop) ----
    // Producer wave p holds, in lane l, channels 2l and 2l+1 of the chunk rows
    // 16p-3 .. 16p+15 of each stream: its block's 16 rows and the three
    // before them, which the causal conv of its first rows reads.  The window
    // then lies within the lane, and each 4-byte load of a wave covers one
    // whole 256-byte token row.  Rows before the sequence's first token come
    // from its FIFO state; rows past its end read its first row (their
    // outputs are zeroed).
    uint32_t raw[3][19];          // bf16 pairs, streams q, k, v
    uint32_t xQ[16], xV[16];      // the block's q (fp16 pairs) and v (bf16 pairs)
    float cw[3][2][4];            // conv weights of channels 2l, 2l+1, taps oldest first

    __device__ void load_weights(const Unit &u, int l) {
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            const float *wp = u.conv_w + ((s * u.H + u.h) * D + 2 * l) * 4;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const f32x4 t = *reinterpret_cast<const f32x4 *>(wp + 4 * c);
#pragma unroll
                for (int j = 0; j < 4; ++j) cw[s][c][j] = t[j];
            }
        }
    }
    // Prefetch of stream s (0 q, 1 k, 2 v) of chunk pc, and of the raw gate
    // inputs a, b of token l.
    __device__ void prefetch_pre(const Unit &u, int pc, int p, int l, int s) {
        const int64_t base = int64_t(pc) * C + 16 * p - 3;   // sequence row of raw[s][0]
        const int64_t HD = u.H * D;
        const uint32_t lo = static_cast<uint32_t>(u.h * D + 2 * l);
        const bf16 *x = s == 0 ? u.q : (s == 1 ? u.k : u.v);
        // the three window rows before the block: FIFO rows at a sequence start
        const bf16 *fifo = u.fifo + ((u.seq * 3 + s) * u.H + u.h) * 3 * D + 2 * l;
#pragma unroll
        for (int j = 0; j < 19; ++j) {
            const int64_t r = base + j;
            const bf16 *ptr;
            if (j < 3 && r < 0)
                ptr = fifo + (3 + r) * D;
            else
                ptr = x + (u.start + (r < u.len ? r : 0)) * HD + lo;
            raw[s][j] = *reinterpret_cast<const uint32_t *>(ptr);
        }
    }
    __device__ void prefetch_gates(const Unit &u, int pc, int l) {
        const int nv = u.rows_in(pc);
        const int64_t gi = (l < nv ? u.row0(pc) + l : u.start) * u.H + u.h;
        pg = u.g[gi];       // raw gate inputs a and b
        pb = u.beta[gi];
    }
    __device__ void prefetch_pre(const Unit &u, int pc, int p, int l) {
#pragma unroll
        for (int s = 0; s < 3; ++s) prefetch_pre(u, pc, p, l, s);
        prefetch_gates(u, pc, l);
    }
    // conv, silu and (for q and k) the row's L2 norm of the stream s rows held
    // in raw[s]; y[r] holds channels 2l, 2l+1 of block row r.
    __device__ void conv_rows(int s, float ceps, float (*y)[2], int l) {
        float x[19][2];
#pragma unroll
        for (int j = 0; j < 19; ++j) {
            x[j][0] = __uint_as_float(raw[s][j] << 16);
            x[j][1] = __uint_as_float(raw[s][j] & 0xffff0000u);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const float u = cw[s][c][0] * x[r][c] + cw[s][c][1] * x[r + 1][c] +
                                cw[s][c][2] * x[r + 2][c] + cw[s][c][3] * x[r + 3][c];
                y[r][c] = u * __builtin_amdgcn_rcpf(1.f + __expf(-u));
            }
        if (s < 2) {
            float ss[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) ss[r] = y[r][0] * y[r][0] + y[r][1] * y[r][1];
            // lane 32 (r >> 3) + 16 ((r >> 2) & 1) + 8 ((r >> 1) & 1) + 4 (r & 1)
            // ends with row r's sum
            const float inv = rsqrtf(rows16_wave_sum(ss, l) + ceps);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int src = 32 * (r >> 3) + 16 * ((r >> 2) & 1) + 8 * ((r >> 1) & 1) + 4 * (r & 1);
                const float f = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, inv), src));
                y[r][0] *= f;
                y[r][1] *= f;
            }
        }
    }
    // The pre-operations on the prefetched rows of a chunk with nv rows:
    // convert_pre_k stores K (fp16) in buffer set nb; convert_pre_qv keeps Q
    // (fp16) and V (bf16) for their stores, and wave p = 0 turns the raw gate
    // inputs into g = -softplus(a), beta = sigmoid(b) and scans them.  Rows
    // past nv are zero.
    __device__ void convert_pre_k(Smem &sm, int nb, int nv, int p, int l, float ceps) {
        typedef f16 f16x2 __attribute__((ext_vector_type(2)));
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        float y[16][2];
        auto live = [&](int r) { return nv >= C || 16 * p + r < nv; };
        conv_rows(1, ceps, y, l);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = 16 * p + r;
            const f16x2 h = live(r) ? __builtin_convertvector(f32x2{y[r][0], y[r][1]}, f16x2) : f16x2{0, 0};
            *reinterpret_cast<f16x2 *>(&sm.K[nb][t * KS + ((2 * l) ^ ksw(t))]) = h;
        }
    }
    __device__ void convert_pre_qv(int nv, int p, int l, float ceps) {
        typedef f16 f16x2 __attribute__((ext_vector_type(2)));
        typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        float y[16][2];
        auto live = [&](int r) { return nv >= C || 16 * p + r < nv; };
        conv_rows(0, ceps, y, l);
#pragma unroll
        for (int r = 0; r < 16; ++r)
            xQ[r] = live(r) ? __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{y[r][0], y[r][1]}, f16x2)) : 0u;
        conv_rows(2, ceps, y, l);
#pragma unroll
        for (int r = 0; r < 16; ++r)
            xV[r] = live(r) ? __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{y[r][0], y[r][1]}, bf16x2)) : 0u;
        if (p == 0) {
            // softplus(a) = max(a, 0) + log1p(exp(-|a|)), without overflow
            pg = -(fmaxf(pg, 0.f) + log1pf(__expf(-fabsf(pg))));
            pb = 1.f / (1.f + __expf(-pb));
            scan(nv, l);
        }
    }
    __device__ void store_v_pre(Smem &sm, int p, int l) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = 16 * p + r;
            *reinterpret_cast<uint32_t *>(&sm.V[t * KS + ((2 * l) ^ ksw(t))]) = xV[r];
        }
    }
    __device__ void store_q_pre(Smem &sm, int nb, int p, int l) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            *reinterpret_cast<uint32_t *>(&sm.Q[nb][(16 * p + r) * QS + 2 * l]) = xQ[r];
        store_scalars(sm, nb, p, l);
    }
    __device__ void store_scalars(Smem &sm, int nb, int p, int l) {
        if (p == 0) {
            sm.G2[nb][l] = sg2;
            sm.EG[nb][l] = seg;
            sm.EC[nb][l] = sec;
            sm.Bt[nb][l] = sbt;
        }
    }


    // Phase 1 for the chunk in buffer set nb: the Gram tiles of row block P of
    // K K^T (-> the diagonal block of N in LDS, the off-diagonal ones kept in
    // Nop) and of column block IB = 3 - P of K Q^T (-> A, kept in Ah).  Masked
    // decay factors take exp2(-inf) = 0 rather than a branch.
    template <int P, bool kHoist>
    __device__ void gram(Smem &sm, int nb, int r16, int q) {
        constexpr int IB = 3 - P;
        constexpr float kNegInf = -__builtin_huge_valf();
        if constexpr (!kHoist) {
            r16 = opaque(r16);
            q = opaque(q);
        }
        const f16 *Kn = sm.K[nb], *Qn = sm.Q[nb];
        const float *G2 = sm.G2[nb], *Bt = sm.Bt[nb];
        constexpr int JM = P > IB ? P : IB;   // K row blocks read: 0..JM
        f32x4 kk[P + 1], qa[IB + 1];
#pragma unroll
        for (int j = 0; j <= P; ++j) kk[j] = zero4();
#pragma unroll
        for (int j = 0; j <= IB; ++j) qa[j] = zero4();
        f16x8 kr[2][JM + 1], qr[2];
        const int kcol = (8 * q) ^ ksw(r16);
        auto ld = [&](int s, f16x8 *k8, f16x8 &q8) {
#pragma unroll
            for (int jb = 0; jb <= JM; ++jb) k8[jb] = rd8(Kn + (16 * jb + r16) * KS + 32 * s + kcol);
            const f16 *qp = Qn + (16 * IB + r16) * QS + 32 * s + 8 * q;
            q8 = cat(rd4(qp), rd4(qp + 4));
        };
        ld(0, kr[0], qr[0]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < 3) ld(s + 1, kr[(s + 1) & 1], qr[(s + 1) & 1]);
            fence();
#pragma unroll
            for (int jb = 0; jb <= P; ++jb) kk[jb] = mfma(kr[s & 1][P], kr[s & 1][jb], kk[jb]);
#pragma unroll
            for (int jb = 0; jb <= IB; ++jb) qa[jb] = mfma(kr[s & 1][jb], qr[s & 1], qa[jb]);
        }
        const f32x4 g2r = *reinterpret_cast<const f32x4 *>(&G2[16 * P + 4 * q]);   // rows 16P + 4q + e
        // kk[jb][e] = k_t . k_j, t = 16P + 4q + e, j = 16jb + r16 (symmetric on
        // the diagonal block).  Diagonal block of N, row u = r16, columns 4q..:
        // N_uj = beta_u exp(G_u - G_j) k_u . k_j for j < u.
        {
            const int u = 16 * P + r16;
            const float g2u = G2[u], bu = Bt[u];
            f32x4 nr;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                nr[e] = bu * (__builtin_amdgcn_exp2f(4 * q + e < r16 ? g2u - g2r[e] : kNegInf) * kk[P][e]);
            *reinterpret_cast<f32x4 *>(&sm.NR[P][r16 * NS + 4 * q]) = nr;
        }
        // Off-diagonal blocks N_Pj (rows t, column j): the A operand of
        // M_Pj^T = N_Pj^T T_PP^T.
        {
            const f32x4 btr = *reinterpret_cast<const f32x4 *>(&Bt[16 * P + 4 * q]);
#pragma unroll
            for (int jb = 0; jb < P; ++jb) {
                const float g2j = G2[16 * jb + r16];
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = btr[e] * (__builtin_amdgcn_exp2f(g2r[e] - g2j) * kk[jb][e]);
                Nop[jb] = split_h4(x);
            }
        }
        // qa[jb][e] = k_j . q_t, j = 16jb + 4q + e, t = 16IB + r16 -> A_tj
        {
            const int t = 16 * IB + r16;
            const float g2t = G2[t];
#pragma unroll
            for (int jb = 0; jb <= IB; ++jb) {
                const f32x4 g2j = *reinterpret_cast<const f32x4 *>(&G2[16 * jb + 4 * q]);
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool keep = jb < IB || 16 * jb + 4 * q + e <= t;
                    x[e] = __builtin_amdgcn_exp2f(keep ? g2t - g2j[e] : kNegInf) * qa[jb][e];
                }
                Ah[jb] = split_h4(x);
            }
        }
    }

    // T_PP = (I + N_PP)^-1 by the exact block doubling of the Qwen3.5-9B-npu
    // model page ("How it works" -> "Gated DeltaNet on the NPU":
    // (D + C)^-1 = D^-1 - D^-1 C D^-1, every intermediate a true
    // sub-inverse).  Starting from D = I, the inverse on the diagonal blocks
    // of size b is extended to size 2b by T <- T - T C_b T, where C_b holds the
    // entries of N coupling the two halves of each 2b block; sizes 2, 4, 8, 16.
    // Each step is three 16x16x16 products on the matrix cores: R = C_b T,
    // T R and its transpose R^T T^T.  T and U = T^T are both kept as result
    // tiles (lane (c = r16, q) holds T[4q+e][c] and T[c][4q+e]): a result tile
    // is a B operand as it is, and read as an A operand it is its own
    // transpose.  Operands are split into fp16 hi + lo pairs, sums are fp32;
    // C_b is taken negated, so that each step accumulates onto T's tiles.
    // Returns the U tile: columns 4q..4q+3 of row r16 of T_PP.
    template <int P>
    __device__ f32x4 invert_doubling(const Smem &sm, int r16, int q) {
        const float *Nr = sm.NR[P];
        const f32x4 nrow = *reinterpret_cast<const f32x4 *>(&Nr[r16 * NS + 4 * q]);   // N[r16][4q..]
        // level 1: T = I - C_1, C_1 = the entries N[i][i-1] of odd rows i
        const float nsub = (r16 & 1) ? 0.f : Nr[(r16 + 1) * NS + r16];               // N[r16+1][r16]
        f32x4 Tt, Ut;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 4 * q + e;
            Tt[e] = (i == r16 ? 1.f : 0.f) - ((r16 & 1) == 0 && i == r16 + 1 ? nsub : 0.f);
            Ut[e] = (i == r16 ? 1.f : 0.f) - ((r16 & 1) == 1 && i == r16 - 1 ? nrow[e] : 0.f);
        }
#pragma unroll
        for (int b = 2; b <= 8; b *= 2) {
            f32x4 cb;   // -C_b[r16][4q+e]: rows in the lower half of a 2b block, columns in its upper half
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * q + e;
                cb[e] = ((r16 / b) & 1) && j / b == r16 / b - 1 ? -nrow[e] : 0.f;
            }
            const h4x2 R = split_h4(prod_split(split_h4(cb), split_h4(Tt), zero4()));   // -C_b T
            const h4x2 uh = split_h4(Ut);
            Tt = prod_split(uh, R, Tt);                                  // T - T C_b T
            Ut = prod_split(R, uh, Ut);                                  // its transpose
        }
        return Ut;
    }

    // Phase 2 for the chunk in buffer set nb: T_PP = (I + N_PP)^-1 by back
    // substitution (row r16 per lane; the four lane groups repeat it) or by
    // block doubling (invert_doubling), T_PP, P_P and P'_P to LDS, and
    // M_Pj = T_PP N_Pj for j < P.
    template <int P, bool kDoubling, bool kHoist>
    __device__ void solve(Smem &sm, int nb, int r16, int q) {
        if constexpr (!kHoist) {
            r16 = opaque(r16);
            q = opaque(q);
        }
        const float *Bt = sm.Bt[nb], *EG = sm.EG[nb];
        f32x4 y4;       // T_PP[r16][4q..4q+3]
        if constexpr (kDoubling) {
            y4 = invert_doubling<P>(sm, r16, q);
        } else {
        // Row r16 of T_PP = (I + N_PP)^-1 by back substitution: y (I + N) = e_t,
        // once y_u is final, y_j -= y_u N_uj for every j < u.  The rows of N
        // are read in three batches (rows 15..12, 11..8, 7..1), each issued
        // before the previous batch is used.
        const float *Nr = sm.NR[P];
        float y[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) y[j] = j == r16 ? 1.f : 0.f;
        f32x4 ra[4][4], rb[4][3], rc[7][2];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4)
                if (4 * v4 < 15 - r) ra[r][v4] = *reinterpret_cast<const f32x4 *>(&Nr[(15 - r) * NS + 4 * v4]);
        fence();
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int v4 = 0; v4 < 3; ++v4)
                if (4 * v4 < 11 - r) rb[r][v4] = *reinterpret_cast<const f32x4 *>(&Nr[(11 - r) * NS + 4 * v4]);
        fence();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int uu = 15 - r;
#pragma unroll
            for (int j = 0; j < uu; ++j) y[j] -= ra[r][j >> 2][j & 3] * y[uu];
        }
        fence();
#pragma unroll
        for (int r = 0; r < 7; ++r)
#pragma unroll
            for (int v4 = 0; v4 < 2; ++v4)
                if (4 * v4 < 7 - r) rc[r][v4] = *reinterpret_cast<const f32x4 *>(&Nr[(7 - r) * NS + 4 * v4]);
        fence();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int uu = 11 - r;
#pragma unroll
            for (int j = 0; j < uu; ++j) y[j] -= rb[r][j >> 2][j & 3] * y[uu];
        }
#pragma unroll
        for (int r = 0; r < 7; ++r) {
            const int uu = 7 - r;
#pragma unroll
            for (int j = 0; j < uu; ++j) y[j] -= rc[r][j >> 2][j & 3] * y[uu];
        }
        // Every lane group holds the whole row; group q keeps columns
        // 4q..4q+3 of it, picked by blending with 0/1 weights (the compiler
        // turns selects on a lane value into an indexed scratch array).
        {
            const float m0 = q == 0 ? 1.f : 0.f, m1 = q == 1 ? 1.f : 0.f;
            const float m2 = q == 2 ? 1.f : 0.f, m3 = q == 3 ? 1.f : 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                y4[e] = y[e] * m0 + y[4 + e] * m1 + y[8 + e] * m2 + y[12 + e] * m3;
        }
        }
        // group q splits and stores its 4 columns of the row
        {
            const f32x4 bt = *reinterpret_cast<const f32x4 *>(&Bt[16 * P + 4 * q]);
            const f32x4 eg = *reinterpret_cast<const f32x4 *>(&EG[16 * P + 4 * q]);
            const int o = r16 * BS + 4 * q;
            const h4x2 ph = split_h4(y4 * (bt * eg));
            const b4x2 pv = split_b4(y4 * bt);
            *reinterpret_cast<f16x4 *>(&sm.P[0][P][o]) = ph.hi;
            *reinterpret_cast<f16x4 *>(&sm.P[1][P][o]) = ph.lo;
            *reinterpret_cast<bf16x4 *>(&sm.Pv[0][P][o]) = pv.hi;
            *reinterpret_cast<bf16x4 *>(&sm.Pv[1][P][o]) = pv.lo;
        }
        // M_Pj^T = N_Pj^T T_PP^T: A = N_Pj (lane: row j = r16, k = t = 4q..),
        // B[t'][t] = T_PP[t][t'] (lane: column t = r16, k = t' = 4q..).  The
        // result lane holds M[t = r16][j = 4q + e]; stored negated, split.
        if (P > 0) {
            const h4x2 tb = split_h4(y4);
#pragma unroll
            for (int jb = 0; jb < P; ++jb) {
                const f32x4 mt = prod_split(Nop[jb], tb, zero4());
                const h4x2 m = split_h4(-mt);
                *reinterpret_cast<f16x4 *>(&sm.M[0][oblk(P, jb)][r16 * BS + 4 * q]) = m.hi;
                *reinterpret_cast<f16x4 *>(&sm.M[1][oblk(P, jb)][r16 * BS + 4 * q]) = m.lo;
            }
        }
    }

    // Phase 3: the A tiles of row block IB = 3 - P of the prepared chunk.
    template <int P>
    __device__ void store_a(Smem &sm, int r16, int q) {
        constexpr int IB = 3 - P;
#pragma unroll
        for (int jb = 0; jb <= IB; ++jb) {
            *reinterpret_cast<f16x4 *>(&sm.A[0][(16 * IB + r16) * AS + 16 * jb + 4 * q]) = Ah[jb].hi;
            *reinterpret_cast<f16x4 *>(&sm.A[1][(16 * IB + r16) * AS + 16 * jb + 4 * q]) = Ah[jb].lo;
        }
    }
};

// Columns [32p, 32p+32) of W and columns [vcol, vcol + 16 NCC) of U for the
// chunk in buffer set nb, block by block (run by consumer wave p); stores -W
// (dk-major) in LDS and returns U in the result-tile layout, Uo[i][cc] = U rows
// 16i + 4q + e, column vcol + 16cc + r16, at the wave's scale for the chunk.
// Every wave forms its 32 columns of W whatever NCC is: the products W S of
// each wave run over all 128 of them.  That scale is chosen here, from the
// largest |X| of the direct terms X_i = P'_i V_i (bf16 products, unscaled) and
// `ms`, the lane's largest |S| at the current scale 2^sc (S being the state
// that enters the chunk); S is rescaled when the scale changes.  W's chain is
// W_i = P_i K_i - sum_j M_ij W_j with P and M split and W single; U's chain
// U_i = X_i - sum_j M_ij U_j with M and U split.
template <int NCC>
__device__ __forceinline__ void wu_step(Smem &sm, int nb, int p, int vcol, f32x4 (*Uo)[NCC],
                                        f32x4 (*S)[NCC], int &sc, float ms) {
    const int lane = fresh_lane_id(), r16 = lane & 15, q = lane >> 4;
    const int trk = (4 * q + (r16 >> 2)) * KS + ((4 * (r16 & 3)) ^ ksw(4 * q));
    const f16 *kb = sm.K[nb] + trk + 32 * p;
    const f16 *vb = reinterpret_cast<const f16 *>(sm.V) + trk + vcol;
    const int co = r16 * BS + 4 * q;
    // Everything but the previous blocks' W and U is known before the
    // substitution starts: read it all first.
    f16x4 kx[4][2];
    bf16x4 vx[4][NCC];
    f16x8 pw[4];
    bf16x8 pu[4];
    h4x2 mm[6];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            kx[i][cc] = rd_tr(kb + 16 * i * KS + 16 * cc);
            if (cc < NCC) vx[i][cc] = __builtin_bit_cast(bf16x4, rd_tr(vb + 16 * i * KS + 16 * cc));
        }
        pw[i] = cat(rd4(&sm.P[0][i][co]), rd4(&sm.P[1][i][co]));
        pu[i] = catb(*reinterpret_cast<const bf16x4 *>(&sm.Pv[0][i][co]),
                     *reinterpret_cast<const bf16x4 *>(&sm.Pv[1][i][co]));
    }
#pragma unroll
    for (int b = 0; b < 6; ++b) mm[b] = h4x2{rd4(&sm.M[0][b][co]), rd4(&sm.M[1][b][co])};
    fence();
    // the direct terms of U, unscaled, and the scale of the chunk
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc) {
            Uo[i][cc] = mfma_bf(pu[i], catb(vx[i][cc], vx[i][cc]), zero4());
            mx = absmax4(Uo[i][cc], mx);
        }
    const int nx = choose_scale(0.f, sc, wave_max_nonneg(fmax_ieee(ms * pow2i(-sc), mx)));
    if (nx != sc) {
        const float f = pow2i(nx - sc);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int cc = 0; cc < NCC; ++cc) S[i][cc] *= f;
        sc = nx;
    }
    const float up = pow2i(sc);
    f16x4 Wr[3][2];
    h4x2 Ur[3][NCC];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f32x4 aw[2], au[NCC];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            aw[cc] = mfma(pw[i], cat(kx[i][cc], kx[i][cc]), zero4());   // P_i K_i
            if (cc < NCC) au[cc] = Uo[i][cc] * up;
        }
        // - M_ij W_j and - M_ij U_j (M is stored negated): the hi products ...
#pragma unroll
        for (int j = 0; j < i; ++j) {
            const h4x2 mj = mm[oblk(i > 0 ? i : 1, j)];
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                aw[cc] = mfma(cat(mj.hi, mj.lo), cat(Wr[j][cc], Wr[j][cc]), aw[cc]);
                if (cc < NCC) au[cc] = mfma(cat(mj.hi, mj.lo), cat(Ur[j][cc].hi, Ur[j][cc].hi), au[cc]);
            }
        }
        // ... and M U_lo: M_hi of two blocks j to a product, or (hi + lo) of one
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc) {
            if (i == 1) {
                au[cc] = mfma(cat(mm[oblk(1, 0)].hi, mm[oblk(1, 0)].lo), cat(Ur[0][cc].lo, Ur[0][cc].lo), au[cc]);
            } else if (i == 2) {
                au[cc] = mfma(cat(mm[oblk(2, 0)].hi, mm[oblk(2, 1)].hi), cat(Ur[0][cc].lo, Ur[1][cc].lo), au[cc]);
            } else if (i == 3) {
                au[cc] = mfma(cat(mm[oblk(3, 0)].hi, mm[oblk(3, 1)].hi), cat(Ur[0][cc].lo, Ur[1][cc].lo), au[cc]);
                au[cc] = mfma(cat(mm[oblk(3, 2)].hi, mm[oblk(3, 2)].lo), cat(Ur[2][cc].lo, Ur[2][cc].lo), au[cc]);
            }
        }
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            const f16x4 w16 = h4(aw[cc]);
            if (i < 3) {
                Wr[i < 3 ? i : 0][cc] = w16;
                if (cc < NCC) Ur[i < 3 ? i : 0][cc] = split_h4(au[cc]);
            }
            *reinterpret_cast<f16x4 *>(&sm.W[(32 * p + 16 * cc + r16) * WS + 16 * i + ((4 * q) ^ wsw(r16))]) = neg(w16);
            if (cc < NCC) Uo[i][cc] = au[cc];
        }
    }
}

template <bool kGated, bool kDoubling, bool kRank, typename OutT, bool kPreop = false, int NCC = 2>
__global__ __launch_bounds__(512) void prefill_mfma_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const float *__restrict__ S0, const int32_t *__restrict__ cu_seqlens, int64_t N, int64_t T,
    int64_t H, OutT *__restrict__ O, float *__restrict__ S_T, const bf16 *__restrict__ z,
    const float *__restrict__ norm_w, float eps, const float *__restrict__ conv_w,
    const bf16 *__restrict__ fifo, float ceps) {
    // NCC = 1: the value columns of each (sequence, head) are split over two
    // workgroups of 64 columns (each consumer wave then owns 16 of them), for
    // launches that would leave most CUs idle.  The columns of S, U, D and O
    // are exactly independent; the producers' work (staging, Gram tiles,
    // inverse) and W are repeated in both workgroups.
    static_assert(NCC == 1 || NCC == 2, "value tiles per consumer wave");
    static_assert(NCC == 2 || (!kGated && !kRank && !kPreop), "split forms");
    __shared__ Smem sm;

    const int tid = threadIdx.x;
    // the wave index is the same in every lane: read it once into a scalar
    // register, so that everything derived from it (roles, column groups, row
    // blocks, LDS offsets) stays scalar instead of taking vector registers.
    // The form with the pre-operations keeps it per lane: there the scalar
    // index measured 8% slower (2.33 against 2.14 ms on the 8 x 16384 x 32
    // prompt), the producers setting that form's period.
    const int wave = kPreop ? (tid >> 6) : __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, r16 = l & 15, qd = l >> 4;
    const int w = wave & 3;                 // consumer column group / producer row block
    // A packed batch of sequences of mixed lengths is walked longest first
    // (in the instantiation the launch picks for it), so that the long ones do
    // not start last and set the end of the launch.
    // Workgroup -> unit (and column half).  The two halves of a unit read the
    // same key and query rows: when the unit count is a multiple of 8 they are
    // workgroups b and b + 8, which the dispatcher's round robin over the 8
    // XCDs puts on the same XCD (and L2).
    int64_t bid = blockIdx.x;
    int half = 0;
    if constexpr (NCC == 1) {
        const uint32_t b = blockIdx.x, units = gridDim.x >> 1;
        if ((units & 7u) == 0) {
            half = (b >> 3) & 1;
            bid = ((b >> 4) << 3) | (b & 7u);
        } else {
            half = b & 1;
            bid = b >> 1;
        }
    }
    int64_t seq = bid / H;
    if constexpr (kRank) {
        // the lengths are staged in the first key buffer, which the producers
        // first write after the barrier below
        static_assert(sizeof(sm.K[0]) >= 4 * (kMaxRankedSequences + 3), "lens buffer");
        __shared__ int64_t pick;
        rank_longest_first(cu_seqlens, N, T, seq, tid, 512, reinterpret_cast<int32_t *>(sm.K[0]),
                           &pick);
        __syncthreads();
        seq = pick;
    }
    const int64_t unit = seq * H + bid % H;
    Unit u;
    u.q = q; u.k = k; u.v = v; u.g = g; u.beta = beta;
    u.H = H;
    u.h = unit % H;
    u.fifo = fifo;
    u.conv_w = conv_w;
    u.seq = seq;
    u.ceps = ceps;
    sequence_span(cu_seqlens, seq, T, u.start, u.len);
    const int nch = static_cast<int>((u.len + C - 1) / C);

    if (wave >= 4) {
        // ======================= producer waves =======================
        if (nch == 0) return;
        // A entries above the diagonal blocks are never written.
        for (int i = (tid - 256) * 8; i < C * AS; i += 256 * 8) {
            *reinterpret_cast<f32x4 *>(&sm.A[0][i]) = zero4();
            *reinterpret_cast<f32x4 *>(&sm.A[1][i]) = zero4();
        }
        Producer pr;
        // Lane-constant masks and offsets of the Gram and inverse steps are
        // hoisted out of the chunk loop (scalar lane masks and a few registers)
        // where the registers allow it; the substitution and pre-operation
        // forms need their registers and recompute them in every period.
        constexpr bool kHoist = kDoubling && !kPreop;
        if constexpr (kPreop) {
            pr.load_weights(u, l);
            pr.prefetch_pre(u, 0, w, l);
            pr.convert_pre_k(sm, 0, u.rows_in(0), w, l, u.ceps);
            pr.convert_pre_qv(u.rows_in(0), w, l, u.ceps);
            pr.store_q_pre(sm, 0, w, l);
            pr.prefetch_pre(u, 1, w, l);
        } else {
            pr.load_k(u, 0, w, r16, qd);
            pr.load_q(u, 0, w, r16, qd);
            pr.load_v(u, 0, w, r16, qd);
            if (w == 0) pr.load_gates(u, 0, l);
            pr.stage_kq(sm, 0, u.rows_in(0), w, l, r16, qd, u, 1);
        }
        __syncthreads();
        // Period c (c = -1 .. nch-1) prepares chunk c+1 and stages chunk c+2;
        // the last period's work is on empty chunks and is never read.
        for (int c = -1; c < nch; ++c) {
            const int nb = (c + 1) & 1;
            if constexpr (kPreop)                      // V of chunk c+1
                pr.store_v_pre(sm, w, l);
            else
                pr.stage_v(sm, u.rows_in(c + 1), w, r16, qd, u, c + 2);
            switch (w) {
            case 0: pr.gram<0, kHoist>(sm, nb, r16, qd); break;
            case 1: pr.gram<1, kHoist>(sm, nb, r16, qd); break;
            case 2: pr.gram<2, kHoist>(sm, nb, r16, qd); break;
            default: pr.gram<3, kHoist>(sm, nb, r16, qd); break;
            }
            __syncthreads();
            // Phase 2's longest work: with the pre-operations the producers'
            // (the inverse chain, then K's conv), which take precedence on
            // their SIMDs (matrix core and vector ALU) until it ends; in the
            // plain form the consumers' output step and the producer of block
            // 3 (its inverse chain and the three M_3j), which alone raises its
            // priority.
            if constexpr (kPreop) {
                __builtin_amdgcn_s_setprio(2);
            } else if constexpr (!kGated) {
                if (w == 3) __builtin_amdgcn_s_setprio(1);
            }
            switch (w) {
            case 0: pr.solve<0, kDoubling, kHoist>(sm, nb, r16, qd); break;
            case 1: pr.solve<1, kDoubling, kHoist>(sm, nb, r16, qd); break;
            case 2: pr.solve<2, kDoubling, kHoist>(sm, nb, r16, qd); break;
            default: pr.solve<3, kDoubling, kHoist>(sm, nb, r16, qd); break;
            }
            // K of chunk c+2 goes to the buffer nobody reads in phases 2 and 3
            if constexpr (kPreop) {
                pr.convert_pre_k(sm, nb ^ 1, u.rows_in(c + 2), w, l, u.ceps);
                pr.prefetch_pre(u, c + 3, w, l, 1);
            }
            if constexpr (!kGated) __builtin_amdgcn_s_setprio(0);
            __syncthreads();
            switch (w) {
            case 0: pr.store_a<0>(sm, r16, qd); break;
            case 1: pr.store_a<1>(sm, r16, qd); break;
            case 2: pr.store_a<2>(sm, r16, qd); break;
            default: pr.store_a<3>(sm, r16, qd); break;
            }
            if constexpr (kPreop) {
                // the pre-operations of chunk c+2's q and v beside the
                // consumers' W/U step, at a raised priority: Q goes to the
                // buffer nobody reads in phase 3, V waits for phase 1
                __builtin_amdgcn_s_setprio(1);
                pr.convert_pre_qv(u.rows_in(c + 2), w, l, u.ceps);
                pr.store_q_pre(sm, nb ^ 1, w, l);
                pr.prefetch_pre(u, c + 3, w, l, 0);
                pr.prefetch_pre(u, c + 3, w, l, 2);
                pr.prefetch_gates(u, c + 3, l);
                __builtin_amdgcn_s_setprio(0);
            } else {
                // K and Q of chunk c+2 staged beside the consumers' W/U step
                // (into the buffers nobody reads in phase 3), and the loads of
                // chunk c+3
                pr.stage_kq(sm, nb ^ 1, u.rows_in(c + 2), w, l, r16, qd, u, c + 3);
            }
            __syncthreads();
        }
        return;
    }

    // ======================= consumer waves =======================
    // S[i][c] holds state rows 16i+4q+e, column col0+16c+r16, at scale 2^sc.
    const int col0 = NCC == 2 ? 32 * w : 64 * half + 16 * w;
    f32x4 S[8][NCC];
    int sc = 0;
    if (S0) {
        const float *S0u = S0 + unit * (D * D);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int c = 0; c < NCC; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    S[i][c][e] = S0u[(16 * i + 4 * qd + e) * D + col0 + 16 * c + r16];
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int c = 0; c < NCC; ++c) S[i][c] = zero4();
    }
    float *STu = S_T + unit * (D * D);
    auto store_state = [&]() {
        const float un = pow2i(-sc);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int c = 0; c < NCC; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    STu[(16 * i + 4 * qd + e) * D + col0 + 16 * c + r16] = S[i][c][e] * un;
    };
    if (nch == 0) {
        store_state();
        return;
    }
    // this lane's largest |S| (at the current scale), for the next scale choice
    auto lane_max_s = [&]() {
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = absmax4(S[i][NCC - 1], absmax4(S[i][0], m));
        return m;
    };
    if (kGated && tid < D) sm.NW[tid] = norm_w[tid];
    if (kGated && tid == 0) sm.NPC = 0;
    __syncthreads();
    // the period in which the producers prepare chunk 0; its phase 3 is the
    // W/U step of chunk 0
    __syncthreads();
    __syncthreads();
    f32x4 Ur[4][NCC];
    wu_step<NCC>(sm, 0, w, col0, Ur, S, sc, lane_max_s());
    __syncthreads();

    const uint32_t HD = static_cast<uint32_t>(H) * D;
    const int trw = (4 * qd + (r16 >> 2)) * WS + ((4 * (r16 & 3)) ^ wsw(4 * qd));
    const int trk = (4 * qd + (r16 >> 2)) * KS + ((4 * (r16 & 3)) ^ ksw(4 * qd));
    for (int c = 0; c < nch; ++c) {
        const int cur = c & 1;
        const int cnv = u.rows_in(c);

        // ======== phase 1: D = U - W S; S <- exp(G_C) S + K^T diag(exp(G_C - G)) D ========
        // (all at the wave's scale: U and S carry it, so D does)
        f16x8 Sh[4][NCC], Dh[2][NCC], Dl[2][NCC];
        {
            const f16 *Wc = sm.W + trw;
            auto ld_w = [&](int s, f16x8 *dst) {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const f16 *wp = Wc + 32 * s * WS + 16 * m;
                    dst[m] = cat(rd_tr(wp), rd_tr(wp + 16 * WS));
                }
            };
            const f16 *Kc = sm.K[cur] + trk;
            auto ld_k = [&](int i, f16x8 *dst) {
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const f16 *kp = Kc + 32 * s2 * KS + 16 * i;
                    dst[s2] = cat(rd_tr(kp), rd_tr(kp + 16 * KS));
                }
            };
            f16x8 wa[2][4];
            ld_w(0, wa[0]);
            f32x4 Dt[4][NCC];
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int cc = 0; cc < NCC; ++cc) Dt[m][cc] = Ur[m][cc];
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int cc = 0; cc < NCC; ++cc) Sh[s][cc] = cat(h4(S[2 * s][cc]), h4(S[2 * s + 1][cc]));
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (s < 3) ld_w(s + 1, wa[(s + 1) & 1]);
                fence();
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int cc = 0; cc < NCC; ++cc) Dt[m][cc] = mfma(wa[s & 1][m], Sh[s][cc], Dt[m][cc]);
            }
            f16x8 ka[2][4];
            ld_k(0, ka[0]);
            ld_k(1, ka[0] + 2);
            fence();
            f16x8 Dp[2][NCC], Dq[2][NCC];   // the decayed D, hi and lo
            const float *EC = sm.EC[cur];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const f32x4 e0 = *reinterpret_cast<const f32x4 *>(&EC[32 * s2 + 4 * qd]);
                const f32x4 e1 = *reinterpret_cast<const f32x4 *>(&EC[32 * s2 + 16 + 4 * qd]);
#pragma unroll
                for (int cc = 0; cc < NCC; ++cc) {
                    const h4x2 d0 = split_h4(Dt[2 * s2][cc]), d1 = split_h4(Dt[2 * s2 + 1][cc]);
                    Dh[s2][cc] = cat(d0.hi, d1.hi);
                    Dl[s2][cc] = cat(d0.lo, d1.lo);
                    const h4x2 p0 = split_h4(Dt[2 * s2][cc] * e0), p1 = split_h4(Dt[2 * s2 + 1][cc] * e1);
                    Dp[s2][cc] = cat(p0.hi, p1.hi);
                    Dq[s2][cc] = cat(p0.lo, p1.lo);
                }
            }
            const float eC = sm.EG[cur][C - 1];
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int cc = 0; cc < NCC; ++cc) S[i][cc] *= eC;
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                if (ib < 3) {
                    ld_k(2 * ib + 2, ka[(ib + 1) & 1]);
                    ld_k(2 * ib + 3, ka[(ib + 1) & 1] + 2);
                }
                fence();
#pragma unroll
                for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                        for (int cc = 0; cc < NCC; ++cc) {
                            S[2 * ib + ii][cc] = mfma(ka[ib & 1][2 * ii + s2], Dp[s2][cc], S[2 * ib + ii][cc]);
                            S[2 * ib + ii][cc] = mfma(ka[ib & 1][2 * ii + s2], Dq[s2][cc], S[2 * ib + ii][cc]);
                        }
            }
        }
        // The largest |S| of the state entering chunk c + 1, for the scale of
        // the next W/U step.  With the gated norm it is taken here and held
        // (the compiler guards that form's reads of state registers with a
        // wait on the vector-memory counter, which in phase 3 would also wait
        // for this chunk's output stores); the other forms take it at the end
        // of phase 2, off the recurrence's chain.
        float msl = 0.f;
        if constexpr (kGated) {
            msl = lane_max_s();
            asm volatile("" : "+v"(msl));
        }
        __syncthreads();

        // ======== phase 2: O = diag(exp G) Q S + A D (S as it entered the chunk) ========
        // Computed transposed, O^T = S^T Q^T diag(exp G) + D^T A^T: the fp16
        // tiles of S and D serve as A operands as they are, a lane's column is
        // one token (one decay factor), and each lane ends up with four
        // consecutive columns of one token row (one 8-byte store).  A D takes
        // both split: (D_hi + D_lo) A_hi + D_hi A_lo.  O is unscaled before it
        // is stored (or normed).
        // With the gated norm, the gate rows z are loaded into registers before
        // the products, O is multiplied by w silu(z) after them, and each wave
        // leaves its partial sums of O^2 per token row in LDS; the four waves
        // meet on an LDS counter and the rows are scaled by
        // 1/sqrt(mean(O^2) + eps) and stored.
        // O rows of the chunk: a base common to the wave (kept in scalar
        // registers) plus one 32-bit byte offset per lane.  No per-lane 64-bit
        // address then has to survive the products, so none is spilled: a
        // reload from scratch would wait for every store the wave has in
        // flight, the output stores included.
        char *const obase = reinterpret_cast<char *>(O + (u.row0(c) * H + u.h) * D);
        const uint32_t olane = (static_cast<uint32_t>(r16) * HD + col0 + 4 * qd) * sizeof(OutT);
        auto orow = [&](int m, int cc) {
            return obase + static_cast<uint32_t>(16 * m) * HD * sizeof(OutT) + olane + 16 * cc * sizeof(OutT);
        };
        f32x4 Ot[4][NCC];         // Ot[m][cc]: O[16m + r16][col0 + 16cc + 4q + e]
        {
            bf16x4 zr[4][NCC];
            if constexpr (kGated) {
                const char *zc = reinterpret_cast<const char *>(z + (u.row0(c) * H + u.h) * D);
                const uint32_t zlane = (col0 + 4 * qd) * sizeof(bf16);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int t = 16 * m + r16;
                    const uint32_t off = static_cast<uint32_t>(t < cnv ? t : 0) * HD * sizeof(bf16) + zlane;
#pragma unroll
                    for (int cc = 0; cc < NCC; ++cc)
                        zr[m][cc] = *reinterpret_cast<const bf16x4 *>(zc + off + 16 * cc * sizeof(bf16));
                }
            }
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int cc = 0; cc < NCC; ++cc) Ot[m][cc] = zero4();
            const f16 *Qc = sm.Q[cur] + r16 * QS + 4 * qd;
            auto ld_q = [&](int s, f16x8 *dst) {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const f16 *qp = Qc + 16 * m * QS + 32 * s;
                    dst[m] = cat(rd4(qp), rd4(qp + 16));
                }
            };
            f16x8 qb[2][4];
            ld_q(0, qb[0]);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (s < 3) ld_q(s + 1, qb[(s + 1) & 1]);
                fence();
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int cc = 0; cc < NCC; ++cc) Ot[m][cc] = mfma(Sh[s][cc], qb[s & 1][m], Ot[m][cc]);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float eg = sm.EG[cur][16 * m + r16];
#pragma unroll
                for (int cc = 0; cc < NCC; ++cc) Ot[m][cc] *= eg;
            }
            {
                const f16 *Ah = sm.A[0] + r16 * AS + 4 * qd, *Al = sm.A[1] + r16 * AS + 4 * qd;
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int s2 = 0; s2 <= m / 2; ++s2) {
                        const f16x8 ah = cat(rd4(Ah + 16 * m * AS + 32 * s2), rd4(Ah + 16 * m * AS + 32 * s2 + 16));
                        const f16x8 al = cat(rd4(Al + 16 * m * AS + 32 * s2), rd4(Al + 16 * m * AS + 32 * s2 + 16));
#pragma unroll
                        for (int cc = 0; cc < NCC; ++cc) {
                            Ot[m][cc] = mfma(Dh[s2][cc], ah, Ot[m][cc]);
                            Ot[m][cc] = mfma(Dl[s2][cc], ah, Ot[m][cc]);
                            Ot[m][cc] = mfma(Dh[s2][cc], al, Ot[m][cc]);
                        }
                    }
            }
            {
                const float un = pow2i(-sc);
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int cc = 0; cc < NCC; ++cc) Ot[m][cc] *= un;
            }
            if constexpr (kGated) {
                const f32x4 nw0 = *reinterpret_cast<const f32x4 *>(&sm.NW[col0 + 4 * qd]);
                const f32x4 nw1 = *reinterpret_cast<const f32x4 *>(&sm.NW[col0 + 16 + 4 * qd]);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    float ss = 0.f;
#pragma unroll
                    for (int cc = 0; cc < NCC; ++cc)
#pragma unroll
                        for (int e = 0; e < 4; ++e) ss += Ot[m][cc][e] * Ot[m][cc][e];
                    // lanes r16 + 16 q of the four lane groups hold one row
                    ss += __shfl_xor(ss, 16);
                    ss += __shfl_xor(ss, 32);
                    if (qd == 0) sm.NP[16 * m + r16][w] = ss;
#pragma unroll
                    for (int cc = 0; cc < NCC; ++cc) {
                        const f32x4 zf = __builtin_convertvector(zr[m][cc], f32x4);
                        const f32x4 nw = cc ? nw1 : nw0;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-zf[e]));
                            Ot[m][cc][e] *= nw[e] * (zf[e] * sg);
                        }
                    }
                }
                // The four consumer waves meet on an LDS counter (the producers
                // are still solving): each posts its partial sums, then waits
                // until all four sets of this chunk are there.  Rows are then
                // normed and stored here.  Every consumer wave posts once per
                // chunk and no wave can run a chunk ahead (the phase barriers),
                // so the count reaches 4 (c + 1); the spin is bounded all the
                // same.
                asm volatile("" ::: "memory");
                __builtin_amdgcn_s_waitcnt(kLgkmcnt0);    // partials landed
                if (l == 0) __hip_atomic_fetch_add(&sm.NPC, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                const uint32_t target = 4u * static_cast<uint32_t>(c + 1);
                for (int spin = 0; spin < (1 << 22); ++spin) {
                    const uint32_t seen = __builtin_amdgcn_readfirstlane(
                        __hip_atomic_load(&sm.NPC, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
                    if (seen >= target) break;
                    __builtin_amdgcn_s_sleep(1);
                }
                asm volatile("" ::: "memory");
                const int rr = opaque(r16);
                const float *np = &sm.NP[rr][0];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const f32x4 ps = *reinterpret_cast<const f32x4 *>(np + 64 * m);
                    const float ms = (ps[0] + ps[1] + ps[2] + ps[3]) * (1.f / D);
                    const float rs = __builtin_amdgcn_rsqf(ms + eps);
                    if (rr < cnv - 16 * m) {
#pragma unroll
                        for (int cc = 0; cc < NCC; ++cc)
                            *reinterpret_cast<bf16x4 *>(orow(m, cc)) = __builtin_convertvector(Ot[m][cc] * rs, bf16x4);
                    }
                }
            } else {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int t = 16 * m + r16;
                    if (O && t < cnv) {
#pragma unroll
                        for (int cc = 0; cc < NCC; ++cc) {
                            if constexpr (sizeof(OutT) == 4)
                                *reinterpret_cast<f32x4 *>(orow(m, cc)) = Ot[m][cc];
                            else
                                *reinterpret_cast<bf16x4 *>(orow(m, cc)) = __builtin_convertvector(Ot[m][cc], bf16x4);
                        }
                    }
                }
            }
        }
        if constexpr (!kGated) msl = lane_max_s();
        __syncthreads();
        // ======== phase 3: W and U of the next chunk ========
        if (c + 1 < nch) wu_step<NCC>(sm, (c + 1) & 1, w, col0, Ur, S, sc, msl);
        __syncthreads();
    }
    store_state();
}

}  // namespace

bool prefill_mfma_supports(const PrefillArgs &a) { return a.bf16 && a.chunk == C; }

// Whether the workgroups of a launch should take their sequences longest first:
// it pays when a packed batch gives each CU only a few workgroups, so that a
// long sequence started late sets the end of the launch; with many short
// workgroups per CU the dispatch balances them already and the ranking (paid
// by every workgroup) only costs.
bool rank_longest_first_pays(const PrefillArgs &a) {
    if (!a.cu_seqlens || a.N > kMaxRankedSequences) return false;
    const int cus = compute_units();
    return cus > 0 && a.N * a.H <= 4 * static_cast<int64_t>(cus);
}

// Whether the value columns of each (sequence, head) should be split over two
// workgroups: when even then the launch's workgroups all run at once (two per
// unit on at most the device's CUs), each unit's chain of chunks then runs on
// two CUs with half the consumer work per chunk.  The gated norm needs a whole
// output row in one workgroup, and the pre-operations would be repeated, so
// those forms are never split.
bool split_columns(const PrefillArgs &a) {
    if (a.z || a.conv_w || 2 * a.N * a.H > int64_t(0x7fffffff)) return false;
    if (a.columns == kColumnsSplit) return true;
    if (a.columns == kColumnsWhole) return false;
    const int cus = compute_units();
    return cus > 0 && 2 * a.N * a.H <= static_cast<int64_t>(cus);
}

template <typename OutT>
void launch_typed(void (*kern)(const bf16 *, const bf16 *, const bf16 *, const float *, const float *,
                               const float *, const int32_t *, int64_t, int64_t, int64_t, OutT *,
                               float *, const bf16 *, const float *, float, const float *,
                               const bf16 *, float),
                  const PrefillArgs &a, hipStream_t stream, int per_unit = 1) {
    const dim3 grid(static_cast<unsigned>(a.N * a.H * per_unit)), block(512);
    kern<<<grid, block, 0, stream>>>(
        static_cast<const bf16 *>(a.q), static_cast<const bf16 *>(a.k),
        static_cast<const bf16 *>(a.v), a.g, a.beta, a.S0, a.cu_seqlens, a.N, a.T, a.H,
        static_cast<OutT *>(a.O), a.S_T, static_cast<const bf16 *>(a.z), a.norm_w, a.eps,
        a.conv_w, static_cast<const bf16 *>(a.fifo), a.ceps);
}

hipError_t launch_prefill_mfma(const PrefillArgs &a, hipStream_t stream) {
    const bool rank = rank_longest_first_pays(a);
    // The inverse method: the caller's, else the default; the plain, gated and
    // fp32-O forms take the same one, so that they share their arithmetic.
    // (The longest-first order is compiled into the default doubling form
    // only; the pre-operations always use doubling: their producers set the
    // period, and substitution there measured 4.0 ms against 2.2 ms on
    // 8 x 16384 x 32.)
    const bool dbl = a.inverse == kInverseDoubling || (a.inverse == kInverseDefault && kDefaultDoubling);
    if (split_columns(a)) {
        if (a.out_f32)
            launch_typed<float>(dbl ? prefill_mfma_kernel<false, true, false, float, false, 1>
                                    : prefill_mfma_kernel<false, false, false, float, false, 1>,
                                a, stream, 2);
        else
            launch_typed<bf16>(dbl ? prefill_mfma_kernel<false, true, false, bf16, false, 1>
                                   : prefill_mfma_kernel<false, false, false, bf16, false, 1>,
                               a, stream, 2);
    } else if (a.conv_w)   // the pre-operations fused into the chunk load
        launch_typed<bf16>(rank ? prefill_mfma_kernel<false, true, true, bf16, true>
                                : prefill_mfma_kernel<false, true, false, bf16, true>, a, stream);
    else if (a.out_f32)
        launch_typed<float>(dbl ? prefill_mfma_kernel<false, true, false, float>
                                : prefill_mfma_kernel<false, false, false, float>, a, stream);
    else if (a.z)
        launch_typed<bf16>(dbl ? prefill_mfma_kernel<true, true, false, bf16>
                               : prefill_mfma_kernel<true, false, false, bf16>, a, stream);
    else if (a.inverse == kInverseDefault && dbl)
        launch_typed<bf16>(rank ? prefill_mfma_kernel<false, true, true, bf16>
                                : prefill_mfma_kernel<false, true, false, bf16>, a, stream);
    else
        launch_typed<bf16>(dbl ? prefill_mfma_kernel<false, true, false, bf16>
                               : prefill_mfma_kernel<false, false, false, bf16>, a, stream);
    return hipGetLastError();
}

}  // namespace gdn
