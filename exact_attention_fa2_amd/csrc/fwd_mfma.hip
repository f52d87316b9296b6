// fwd_mfma.hip -- exact attention forward, f16 / bf16 in and out, D = 64 or
// 128, on gfx950 matrix cores (v_mfma_f32_32x32x16_{f16,bf16}; shapes with
// few tiles also v_mfma_f32_16x16x32, in 16-row waves), f32 softmax state.
//
// Method: the FlashAttention-2 forward ("Flash Attention" (aarnphm.xyz),
// sections Deriving the online softmax and FlashAttention 2; "06: Fused
// attention", attn_fwd).  A workgroup owns 128 query rows, one 32-row slab per
// wave (each wave owns whole rows, so no cross-wave reduction is needed), or
// 256 rows with two slabs per wave (QG = 2, half the LDS reads per flop) when
// the tiles fill the device in whole rounds, and walks the keys in blocks of
// 64 staged through LDS; with few tiles the keys are also cut into chunks
// whose partial states the combine kernel merges, or, with two chunks, the
// second workgroup of the pair to finish.  Per block and wave:
//     S^T = K Q^T                    (D/8 MFMAs, f32 accumulate)
//     m_new = max(m, rowmax S);  P = exp(S - m);  l = l*corr + rowsum P
//     O^T = corr*O^T + V^T P^T       (D/8 MFMAs, P rounded to the input dtype)
// After the last block O = O/l is rounded to the output dtype and
// LSE = m + ln l is stored.  Causal: blocks wholly above the diagonal are never
// loaded, blocks wholly above one wave's rows are skipped by that wave, and
// only blocks that cross the diagonal are masked ("Flash Attention", note on
// causal masking).
//
// Schedule (gfx950-specific):
//   * K and V blocks move HBM/L2 -> LDS with buffer loads that write LDS
//     directly (no registers, no LDS store instructions), double-buffered, so
//     one barrier per block suffices and block j+2's K and block j+1's V are
//     in flight while block j is computed.
//   * The scores of block j+1 are issued to the matrix cores before the
//     softmax of block j runs on the vector ALUs, so the two overlap in one
//     wave (the FlashAttention-3 idea of hiding softmax under the other GEMM,
//     "Flash Attention", section FlashAttention 3).
//   * Rescaling is conditional ("Flash Attention", section FlashAttention 4):
//     the running max used for the exponentials only moves when a row's max
//     grows by more than 2^8, so exp(S - m) stays <= 256 and the O rescale is
//     skipped almost always.  The result is unchanged: O and l carry the same
//     factor and LSE = m + ln l holds for any m used consistently.
//   * Two row sums are kept: l from the f32 values of P, which gives the LSE
//     its float32 accuracy, and lt from P as rounded for the MFMA (dot2 with
//     ones), which normalises O, so O = sum(P~ V) / sum(P~) is exactly the
//     convex combination with the weights the matrix cores used.  When one
//     key dominates a row this cancels the rounding of its weight.
//
// Register layouts (32x32 MFMA accumulator: lane l, register r holds row
// 8*(r/4) + 4*(l/32) + r%4, column l%32):
//   * S^T has keys as rows and queries as columns: lane l holds 32 scores of
//     ONE query (l%32); its partner lane l^32 holds the other 32.
//   * O^T likewise holds half of the D output columns of that query, so corr
//     and 1/l are per-lane scalars.
//   * The P registers feed the B operand of O^T = V^T P^T without moving:
//     16-key chunk c of key tile T uses registers 8c..8c+7 of tile T.  The
//     matching V^T operand comes from the row-major V block by the transposed
//     LDS read (ds_read_b64_tr_b16): lane i of each 16-lane group receives 4
//     keys of d = i when the group points at 4 keys x 4 groups of 4 columns.
//   * LDS rows (2D bytes) have their 16-byte chunks XOR-swizzled by key.
#include <algorithm>
#include <type_traits>

#include "fa2_device.h"
#include "fa2_internal.h"

namespace fa2 {

namespace {

constexpr int kBR = 128;     // query rows per workgroup with one query group per wave
constexpr int kBC = 64;      // keys per block
constexpr int kWaves = 4;    // waves per workgroup
// A tile is accepted with the current running max when each lane's sum of its
// 16 rounded P values is at most this (so every P <= 2^8, far below the f16
// and bf16 overflow); otherwise the max is taken and O rescaled.
constexpr float kLazyCap = 256.f;

// Tuning knobs (compile-time).  FA2_KSWZ selects the K-tile chunk swizzle:
// 1 = chunk ^ ((key/2) % 8), conflict-free for 16 lanes x 16 bytes over 64
// banks; 0 = chunk ^ (key % 8).  FA2_SGB pins the issue order inside a tile
// (score MFMAs interleaved with the exponentials) with scheduling barriers:
// 0 never, 1 always, 2 with D = 128 only (at D = 64 the compiler's own order
// measured about 1% faster, at D = 128 the pinned one about 0.5%).
#ifndef FA2_KSWZ
#define FA2_KSWZ 1
#endif
#ifndef FA2_SGB
#define FA2_SGB 2
#endif
// FA2_VSWZ selects the V-tile swizzle (V is only read transposed, 32 lanes x
// 8 bytes per pass over 4 consecutive keys): 1 = chunk ^ (j ^ 4(j % 2)) with
// j = (key/2) % 8, under which keys k and k + 2 differ in bit 2 and the read
// has no bank conflicts; 0 = chunk ^ (key % 8) (2-way conflicts).
#ifndef FA2_VSWZ
#define FA2_VSWZ 1
#endif

// With D = 128 a row spans all 64 banks and both tiles use chunk ^ (4(key %
// 4) + (key / 4) % 4): a permutation of the 16 chunks over any 16 keys (row
// reads) that moves 4 consecutive keys to different aligned groups of four
// chunks (transposed reads).
template <int D>
__device__ __forceinline__ int kswz(int key) {
    if constexpr (D == 128) return ((key & 3) << 2) | ((key >> 2) & 3);
    return FA2_KSWZ ? (key >> 1) & 7 : key & 7;
}
template <int D>
__device__ __forceinline__ int vswz(int key) {
    if constexpr (D == 128) return ((key & 3) << 2) | ((key >> 2) & 3);
    const int j = (key >> 1) & 7;
    return FA2_VSWZ ? j ^ ((j & 1) << 2) : key & 7;
}

// FA2_POLY_EXP = k (0..8): in every 32-key tile, k of each group's 8 pairs of
// exponentials are computed by exp2_poly on the FMA path instead of by
// v_exp_f32 -- the FlashAttention-4 lever of running a polynomial exponential
// beside the hardware one ("Flash Attention", section FlashAttention 4).  The
// pairs are spread evenly over the tile.  On gfx950 both run on the same
// vector ALU (v_exp_f32 costs about three FMA issue slots), so the product
// build uses 0; a build with k > 0 exists to measure that in the kernel.
#ifndef FA2_POLY_EXP
#define FA2_POLY_EXP 0
#endif

// 2^x = 2^n 2^f with n = floor(x), f = x - n in [0, 1) (exact in f32), and
// 2^f from a cubic whose coefficients were fitted here to the least maximum
// relative error on [0, 1) (8.6e-5 in f32 arithmetic, below the half-ulp of
// the f16 and bf16 P it feeds).  x is clamped at -128, where the result is
// 2^-128: zero once P is rounded to f16, and below 1e-38 in bf16.
__device__ __forceinline__ float exp2_poly(float x) {
    x = fmaxf(x, -128.f);
    const float n = __builtin_floorf(x);
    const float f = x - n;
    const float p = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(0.07706704f, f, 0.22764499f), f,
                                                  0.69511676f),
                                   f, 1.f);
    return __builtin_ldexpf(p, (int)n);
}

// max over the two lanes l and l^32 of a wave (v_permlane32_swap exchanges the
// halves of a register pair; either output pairing gives both halves).
__device__ __forceinline__ float max_halves(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

template <int DT>
struct MfmaT;
template <>
struct MfmaT<1> {
    static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                                      __builtin_bit_cast(half8, b), c, 0, 0, 0);
    }
};
template <>
struct MfmaT<2> {
    static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

// QG: query groups of 32 rows per wave (1 or 2).  With QG = 2 a wave owns 64
// rows, every K and V fragment it reads from LDS feeds two MFMAs, and the
// LDS reads per flop halve (the kernel then runs two waves per SIMD instead of
// three).
// SPLIT: the key blocks of each query tile are cut into gridDim.y chunks, one
// per workgroup along y ("Flash decoding": split the keys, keep unnormalised
// partials); the workgroup writes, per row and chunk, O_s (not divided),
// m_s (natural-log units), the denominator of the rounded P (lt, which
// normalises O) and, with WLSE, that of the f32 P (l, for the LSE), and the
// combine kernel merges them.  With tags (gridDim.y = 2) the two workgroups
// of a tile merge their states themselves: each publishes its state with
// system-scope stores and swaps the launch's tag into tags[blockIdx.x]; the
// one that finds the tag already there merges both in chunk order and writes
// O and LSE (no combine launch).
// D: head dimension, 64 or 128 (128 only with QG = 1: its Q operand and O
// accumulator take twice the registers, and its K/V buffers 64 KB of LDS).
template <int D, int DT, bool CAUSAL, bool WLSE, bool SPLIT, int QG>
__global__ __launch_bounds__(kWaves * 64, QG == 1 && D == 64 ? 3 : 2) void fwd_mfma_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, uint16_t *__restrict__ O, float *__restrict__ LSE,
    float *__restrict__ o_part, float *__restrict__ m_part, float *__restrict__ l_part,
    float *__restrict__ l2_part, unsigned long long *__restrict__ tags, unsigned long long tag,
    int Nq, int Nk, float scale_log2, int n_qtiles, int n_tiles, int snake) {
    static_assert((D == 64 || D == 128) && (D == 64 || QG == 1), "head dimension");
    constexpr int kD = D;
    constexpr int NC = D / 16;                      // 16-wide contraction chunks of S^T = K Q^T
    constexpr int NT = D / 32;                      // 32-column tiles of O^T
    constexpr int CPR = D / 8;                      // 16-byte chunks per LDS row
    constexpr int UPL = kBC * CPR / (kWaves * 64);  // 16-byte DMA units per lane per block
    constexpr int ROWS = kWaves * 32 * QG;          // query rows per workgroup
    // Two K and two V buffers of 64 rows, as separate arrays (not one indexed
    // array) so the compiler can see that reads of one never alias DMA into
    // another.  V buffer b holds keys [64b, 64b + 64) of its block; K buffer b
    // holds keys [64b + 32, 64b + 96), one 32-key tile later, because the
    // scores of tile t + 1 are computed while tile t is consumed.
    __shared__ __attribute__((aligned(16))) uint16_t sK0[kBC * kD];
    __shared__ __attribute__((aligned(16))) uint16_t sK1[kBC * kD];
    __shared__ __attribute__((aligned(16))) uint16_t sV0[kBC * kD];
    __shared__ __attribute__((aligned(16))) uint16_t sV1[kBC * kD];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;
    const int ql = lane & 31;

    // Workgroups go round-robin to the 8 XCDs (and, within one, to its shader
    // engines).
    int bh, qt;
    if (CAUSAL && snake > 0) {
        // Causal grid within one round of slots: the p-th workgroup sent to
        // an XCD lands on its CU p % snake in round p / snake.  Rank the
        // XCD's tiles by length (longest first) and deal ranks to the CUs in
        // a snake -- forward in even rounds, backward in odd ones -- so each
        // CU's tiles add up to about the same number of key blocks (handing
        // out longest first would give one CU the longest tile of three
        // heads).  The host checks that heads do not straddle XCDs.
        const int per_xcd = n_tiles >> 3, hpx = per_xcd / n_qtiles;
        const int xcd = blockIdx.x & 7, pos = blockIdx.x >> 3;
        const int r = pos / snake, i = pos - r * snake;
        const int cnt = min(snake, per_xcd - r * snake);  // workgroups in this round
        const int k = r * snake + ((r & 1) ? cnt - 1 - i : i);
        qt = n_qtiles - 1 - k / hpx;
        bh = xcd * hpx + k % hpx;
    } else if (CAUSAL) {
        // b*h varies fastest and the longest tiles go first: workgroups that
        // arrive together have the same length, so the XCDs, and the shader
        // engines within each, all get the same mix of lengths.  With b*h a
        // multiple of 8, each XCD sees only every eighth head.
        const int n_bh = n_tiles / n_qtiles;
        const int rank = (int)blockIdx.x / n_bh;
        qt = n_qtiles - 1 - rank;
        bh = (int)blockIdx.x - rank * n_bh;
    } else {
        // Unmasked tiles all have the same length: give each XCD a contiguous
        // run of tiles so the query tiles of one head share that XCD's L2.
        int wg = blockIdx.x;
        if ((n_tiles & 7) == 0) wg = (wg & 7) * (n_tiles >> 3) + (wg >> 3);
        bh = wg / n_qtiles;
        qt = wg - bh * n_qtiles;
    }
    const int q0 = qt * ROWS;
    const int qw = q0 + wave * 32 * QG;  // first row of this wave; group g starts at qw + 32g

    const uint16_t *Qh = Q + (size_t)bh * Nq * kD;
    const uint16_t *Kh = K + (size_t)bh * Nk * kD;
    const uint16_t *Vh = V + (size_t)bh * Nk * kD;
    const auto rq = make_rsrc(Qh, (uint32_t)Nq * kD * 2);
    const auto rk = make_rsrc(Kh, (uint32_t)Nk * kD * 2);
    const auto rv = make_rsrc(Vh, (uint32_t)Nk * kD * 2);

    // The loop below takes row maxima of the unscaled scores and masks keys
    // with -inf before the scale is applied, which holds for a positive scale
    // only.  A negative scale is moved onto Q (an exact sign flip) and a zero
    // scale becomes Q = 0 with scale 1: the scaled scores are the same.  (Q is
    // changed after the prologue's wait for its loads, so that its latency
    // still overlaps the first K/V copies.)
    const uint32_t qflip = scale_log2 < 0.f ? 0x80008000u : 0u;
    const uint32_t qkeep = scale_log2 == 0.f ? 0u : 0xFFFFFFFFu;
    scale_log2 = scale_log2 == 0.f ? 1.f : fabsf(scale_log2);

    // B operand of S^T = K Q^T for group g: chunk dc, slot (h, j) is
    // Q[qw + 32g + ql][16dc + 8h + j].
    u32x4 qf[QG][NC];
#pragma unroll
    for (int g = 0; g < QG; ++g)
#pragma unroll
        for (int dc = 0; dc < NC; ++dc)
            qf[g][dc] = load16(rq, (uint32_t)(((qw + 32 * g + ql) * kD + 16 * dc + 8 * h) * 2));

    const int kend = CAUSAL ? min(Nk, q0 + ROWS) : Nk;
    const int nblk = (kend + kBC - 1) / kBC;  // 64-key V blocks of this query tile
    // This workgroup's blocks [b0, b1): all of them, or its chunk of them.
    int b0 = 0, b1 = nblk;
    if constexpr (SPLIT) {
        const int nb = (nblk + (int)gridDim.y - 1) / (int)gridDim.y;
        b0 = min(nblk, (int)blockIdx.y * nb);
        b1 = min(nblk, b0 + nb);
    }
    // Last 32-key tile this wave needs (causal: the one holding the diagonal
    // of its last row group).
    const int t_last = CAUSAL ? min((kend + 31) / 32 - 1, (qw + 32 * (QG - 1)) / 32) : 2 * nblk - 1;

    // Rows past Nk are never loaded with data; make sure the V rows they
    // would occupy hold zeros (0 * V must stay 0 for the masked keys).
    if (Nk % kBC != 0) {
        u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < UPL; ++i) {
            reinterpret_cast<u32x4 *>(sV0)[tid + 256 * i] = z;
            reinterpret_cast<u32x4 *>(sV1)[tid + 256 * i] = z;
        }
        __syncthreads();
    }

    // HBM/L2 -> LDS of the 64 rows starting at key k0: wave w moves 16-byte
    // units [(UPL w + i) 64, +64) of the block; unit P holds chunk (P % CPR) ^
    // swizzle(row) of row P / CPR (kswz for K, vswz for V).  Rows before key
    // 0 or past Nk are out of the descriptor's range and load nothing.
    auto dma = [&](const __amdgpu_buffer_rsrc_t &r, uint16_t *dst, int k0, bool r_is_k) {
#pragma unroll
        for (int i = 0; i < UPL; ++i) {
            const int unit = (UPL * wave + i) * 64 + lane;
            const int row = unit / CPR;
            const int ch = (unit % CPR) ^ (r_is_k ? kswz<D>(row) : vswz<D>(row));
            const int key = k0 + row;
            const uint32_t off = key < 0 ? 0xFFFFFFF0u : (uint32_t)((key * kD + ch * 8) * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst + (UPL * wave + i) * 512), 16,
                                                     off, 0, 0, 0);
        }
    };
    // The same for k0 >= 0 through a descriptor that starts at key k0 and
    // covers the keys left (none past Nk): the per-lane offsets do not
    // change from block to block, and the block's position is scalar work.
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // for the LDS destinations
    auto dma_at = [&](const uint16_t *X, uint16_t *dst, int k0, bool r_is_k) {
        const int kb = k0 < Nk ? k0 : Nk;  // base within the tensor; no records past Nk
        const auto r = make_rsrc(X + (size_t)kb * kD, (uint32_t)(Nk - kb) * kD * 2);
#pragma unroll
        for (int i = 0; i < UPL; ++i) {
            const int unit = (UPL * wave + i) * 64 + lane;
            const int row = unit / CPR;
            const int ch = (unit % CPR) ^ (r_is_k ? kswz<D>(row) : vswz<D>(row));
            const uint32_t off = (uint32_t)((row * kD + ch * 8) * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst + (UPL * wave_s + i) * 512), 16,
                                                     off, 0, 0, 0);
        }
    };

    // LDS offsets that do not change from tile to tile (relative to the
    // tile's first row; both halves of a 64-row buffer share the swizzle).
    int kofs[NC], vofs[NT][2];  // vofs[dt][u]: keys kl (u = 0) and kl + 8 (u = 1)
#pragma unroll
    for (int dc = 0; dc < NC; ++dc) kofs[dc] = ql * kD + (((2 * dc + h) ^ kswz<D>(ql)) << 3);
    {
        const int i = lane & 15;
        const int kl = 4 * h + (i >> 2);
#pragma unroll
        for (int dt = 0; dt < NT; ++dt) {
            const int d = 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (i & 3);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int key = kl + 8 * u;
                vofs[dt][u] = key * kD + (((d >> 3) ^ vswz<D>(key)) << 3) + (d & 7);
            }
        }
    }

    float m[QG], l[QG], lt[QG];  // per group: max used for the exponentials (base 2) and
                                 // this lane's halves of the denominators (f32 P, rounded P)
    const uint32_t ones = DT == 1 ? 0x3C003C00u : 0x3F803F80u;  // (1, 1) in f16 / bf16
    f32x16 oacc[QG][NT];
#pragma unroll
    for (int g = 0; g < QG; ++g) {
        m[g] = -INFINITY;
        l[g] = lt[g] = 0.f;
#pragma unroll
        for (int dt = 0; dt < NT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[g][dt][i] = 0.f;
    }

    // One 32-key tile t.  On entry scur[g] holds S^T of tile t for group g
    // (lane: query qw + 32g + ql, register r: key 32t + 8(r/4) + 4h + r%4),
    // kn points at the LDS rows of tile t+1's keys and vt at those of tile t's
    // values.  With NEXT, the scores of tile t+1 go to snext; the matrix cores
    // run them while the vector ALUs compute this tile's exponentials.
    auto tile = [&](const int t, const uint16_t *kn, const uint16_t *vt, f32x16 *scur,
                    f32x16 *snext, auto next_tag) {
        constexpr bool NEXT = decltype(next_tag)::value;
        const int k0 = 32 * t;
        // All LDS operands of this tile, issued first so their latency is
        // covered by the exponentials.
        u32x4 kf[NC];
        if constexpr (NEXT) {
#pragma unroll
            for (int dc = 0; dc < NC; ++dc) kf[dc] = *reinterpret_cast<const u32x4 *>(&kn[kofs[dc]]);
        }
        u32x4 vf[2][NT];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int dt = 0; dt < NT; ++dt) {
                const uint16_t *src = vt + 16 * c * kD;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(src + vofs[dt][0]));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(src + vofs[dt][1]));
                const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
                const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
                vf[c][dt] = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
            }

        const bool need_mask = (k0 + 32 > Nk) || (CAUSAL && k0 + 31 > qw);
        if (need_mask) {
#pragma unroll
            for (int g = 0; g < QG; ++g)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 8 * (r >> 2) + 4 * h + (r & 3);
                    bool ok = key < Nk;
                    if (CAUSAL) ok = ok && key <= qw + 32 * g + ql;
                    if (!ok) scur[g][r] = -INFINITY;
                }
        }
        // P = exp2(S*scale*log2e - m) of group g for this tile, rounded for
        // the MFMA (pk), with its row sums (lp from the rounded P, ps from f32 P).
        u32x4 pk[QG][2];
        float ps[QG][2], lp[QG][2];
        auto exps = [&](int g, float m_use, bool with_next) __attribute__((always_inline)) {
            ps[g][0] = ps[g][1] = lp[g][0] = lp[g][1] = 0.f;
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 8 * c + 2 * j;
                    const float x0 = __builtin_fmaf(scur[g][r], scale_log2, -m_use);
                    const float x1 = __builtin_fmaf(scur[g][r + 1], scale_log2, -m_use);
                    const bool poly = FA2_POLY_EXP > 0 && ((4 * c + j) * FA2_POLY_EXP) % 8 < FA2_POLY_EXP;
                    const float p0 = poly ? exp2_poly(x0) : exp2f_fast(x0);
                    const float p1 = poly ? exp2_poly(x1) : exp2f_fast(x1);
                    const uint32_t w = pack2<DT>(p0, p1);
                    pk[g][c][j] = w;
                    if constexpr (WLSE) ps[g][j & 1] += p0 + p1;
                    lp[g][j & 1] = dot2<DT>(w, ones, lp[g][j & 1]);
                    if constexpr (NEXT) {
                        // scores of the next tile, one MFMA per exponential pair
                        // of chunk 0 (D = 64) or of both chunks (D = 128)
                        if (with_next && (NC == 8 || c == 0)) {
                            const int jj = NC == 8 ? 4 * c + j : j;
                            snext[g] = MfmaT<DT>::mma(kf[jj], qf[g][jj], jj == 0 ? f32x16{} : snext[g]);
                        }
                    }
                }
        };
        // The running max m is only moved when it must be ("Flash Attention",
        // FlashAttention 4: conditional rescaling).  First try the current m:
        // if every lane's sum of this tile's rounded P is at most 2^8, every P
        // is, and the tile is done without computing its max.  Otherwise (and
        // on a row's first tile, where m is still -inf) take the max, rescale
        // O and the sums, and redo the exponentials.
#pragma unroll
        for (int g = 0; g < QG; ++g) exps(g, m[g] == -INFINITY ? 0.f : m[g], true);
#if FA2_SGB
        if constexpr (NEXT && QG == 1 && (FA2_SGB == 1 || D == 128)) {
#pragma unroll
            for (int j = 0; j < NC; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x002, (WLSE ? 32 : 24) / NC, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
        }
#endif
#pragma unroll
        for (int g = 0; g < QG; ++g) {
            if (__builtin_amdgcn_ballot_w64(m[g] == -INFINITY || lp[g][0] + lp[g][1] > kLazyCap) != 0) {
                float mx = -INFINITY;
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, scur[g][r]);
                mx = max_halves(mx) * scale_log2;
                const float m_new = fmaxf(m[g], mx);
                const float m_use = m_new == -INFINITY ? 0.f : m_new;
                const float corr = exp2f_fast(m[g] - m_use);
                l[g] *= corr;
                lt[g] *= corr;
#pragma unroll
                for (int dt = 0; dt < NT; ++dt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[g][dt][i] *= corr;
                m[g] = m_new;
                exps(g, m_use, false);
            }
        }
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int g = 0; g < QG; ++g)
#pragma unroll
                for (int dt = 0; dt < NT; ++dt)
                    oacc[g][dt] = MfmaT<DT>::mma(vf[c][dt], pk[g][c], oacc[g][dt]);
#pragma unroll
        for (int g = 0; g < QG; ++g) {
            lt[g] += lp[g][0] + lp[g][1];
            if constexpr (WLSE) l[g] += ps[g][0] + ps[g][1];
        }
    };

    auto run_tile = [&](const int t, const uint16_t *kn, const uint16_t *vt, f32x16 *scur,
                        f32x16 *snext) {
        if constexpr (CAUSAL) {
            if (t > t_last) return;
            if (t + 1 <= t_last)
                tile(t, kn, vt, scur, snext, std::true_type{});
            else
                tile(t, kn, vt, scur, snext, std::false_type{});
        } else {
            tile(t, kn, vt, scur, snext, std::true_type{});
        }
    };

    // One 64-key V block b (tiles 2b, 2b+1).  On entry V block b is in vc and
    // K buffer kc holds keys [64b + 32, 64b + 96) (tiles 2b+1 and 2b+2);
    // block b+1 streams into vd / kd, last read in block b-1.
    auto block = [&](int b, const uint16_t *kc, uint16_t *kd, const uint16_t *vc, uint16_t *vd,
                     f32x16 *sa, f32x16 *sb) {
        if (b + 1 < b1) {
            dma_at(Vh, vd, (b + 1) * kBC, false);
            dma_at(Kh, kd, (b + 1) * kBC + 32, true);
        }
        run_tile(2 * b, kc, vc, sa, sb);
        run_tile(2 * b + 1, kc + 32 * kD, vc + 32 * kD, sb, sa);
        // This block's DMA has landed; after the barrier every wave's has.
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
    };

    // Prologue: V block b0, K buffer 0 (keys 64 b0 + 32 .. + 95) and, in K
    // buffer 1's upper half, keys 64 b0 .. + 31; the scores of tile 2 b0; then
    // a barrier so that K buffer 1 may be refilled.  (b0 and b1 are the same
    // for every wave, so all of them take the same branches to the barriers.)
    if (b0 < b1) {
        dma(rv, sV0, b0 * kBC, false);
        dma(rk, sK0, b0 * kBC + 32, true);
        dma(rk, sK1, b0 * kBC - 32, true);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
#pragma unroll
        for (int g = 0; g < QG; ++g)
#pragma unroll
            for (int dc = 0; dc < NC; ++dc) qf[g][dc] = (qf[g][dc] ^ qflip) & qkeep;
        f32x16 sa[QG], sb[QG];
#pragma unroll
        for (int dc = 0; dc < NC; ++dc) {
            const u32x4 a = *reinterpret_cast<const u32x4 *>(&sK1[32 * kD + kofs[dc]]);
#pragma unroll
            for (int g = 0; g < QG; ++g) sa[g] = MfmaT<DT>::mma(a, qf[g][dc], dc == 0 ? f32x16{} : sa[g]);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        // Unrolled by 2 so every buffer and register choice is fixed at compile time.
        for (int b = b0; b < b1; b += 2) {
            block(b, sK0, sK1, sV0, sV1, sa, sb);
            if (b + 1 < b1) block(b + 1, sK1, sK0, sV1, sV0, sa, sb);
        }
    }

    // oacc[g][dt][r] = O[qw + 32g + ql][32dt + 8(r/4) + 4h + r%4] * lt[g]
#pragma unroll
    for (int g = 0; g < QG; ++g) {
        lt[g] += __shfl_xor(lt[g], 32);
        if constexpr (WLSE) l[g] += __shfl_xor(l[g], 32);
    }
    if constexpr (SPLIT) {
        // Partials: stage 32 rows x D columns at a time in LDS (each wave its
        // own buffer of 64 D 2 bytes, free after the last barrier) so that each
        // row's 4D bytes go out as one contiguous piece.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        float *stage = reinterpret_cast<float *>(wave == 0 ? sK0 : wave == 1 ? sK1 : wave == 2 ? sV0 : sV1);
        // Group g's unnormalised O into the wave's stage: row ql, columns
        // swizzled by 4 (ql % 8) so that the rows' f32x4 reads do not conflict.
        auto stage_o = [&](int g) __attribute__((always_inline)) {
#pragma unroll
            for (int dt = 0; dt < NT; ++dt)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int r = 4 * g4;
                    *reinterpret_cast<f32x4 *>(stage + ql * kD + ((32 * dt + 8 * g4 + 4 * h) ^ (4 * (ql & 7)))) =
                        f32x4{oacc[g][dt][r], oacc[g][dt][r + 1], oacc[g][dt][r + 2], oacc[g][dt][r + 3]};
                }
        };
        if (tags) {
            // The pair's states, per (tile, chunk) one block of PF floats:
            // O [ROWS][D], then m (base 2), lt and l per row.  Stores and
            // loads use cache policy 17 (SC0 | SC1, system scope), so the
            // partner reads them from memory whichever XCD it runs on; the
            // tag swap follows this workgroup's last completed store.
            constexpr int kSys = 17;
            constexpr int PF = ROWS * (kD + 3);
            const int chunk = blockIdx.y;
            const auto rmine = make_rsrc(o_part + ((size_t)blockIdx.x * 2 + chunk) * PF, PF * 4);
            const auto rother = make_rsrc(o_part + ((size_t)blockIdx.x * 2 + (chunk ^ 1)) * PF, PF * 4);
#pragma unroll
            for (int g = 0; g < QG; ++g) {
                const int rl = wave * 32 * QG + 32 * g;  // group g's first row within the tile
                stage_o(g);
                if (h == 0) {
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m[g]), rmine, (ROWS * kD + rl + ql) * 4, 0, kSys);
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lt[g]), rmine,
                                                          (ROWS * kD + ROWS + rl + ql) * 4, 0, kSys);
                    if constexpr (WLSE)
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l[g]), rmine,
                                                              (ROWS * kD + 2 * ROWS + rl + ql) * 4, 0, kSys);
                }
#pragma unroll
                for (int j = 0; j < 8; ++j)
#pragma unroll
                    for (int hc = 0; hc < D / 64; ++hc) {
                        const int row = 4 * j + (lane >> 4);
                        const int col = 64 * hc + 4 * (lane & 15);
                        const f32x4 val =
                            *reinterpret_cast<const f32x4 *>(stage + row * kD + (col ^ (4 * (row & 7))));
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, val), rmine,
                                                               ((rl + row) * kD + col) * 4, 0, kSys);
                    }
            }
            __shared__ int s_second;
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (tid == 0) {
                const unsigned long long old =
                    __hip_atomic_exchange(&tags[blockIdx.x], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                const int second = old == tag;
                if (second)  // ready for the next launch
                    __hip_atomic_exchange(&tags[blockIdx.x], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                s_second = second;
            }
            __syncthreads();
            if (!s_second) return;

            // Second: per row the weights of the two states (lane ql, either
            // half, holds row ql's), then O in chunk order -- the same
            // arithmetic whichever workgroup of the pair does it.
            const bool c0 = chunk == 0;
#pragma unroll
            for (int g = 0; g < QG; ++g) {
                const int rl = wave * 32 * QG + 32 * g;
                const float mo = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rother, (ROWS * kD + rl + ql) * 4, 0, kSys));
                const float lto = __uint_as_float(
                    __builtin_amdgcn_raw_buffer_load_b32(rother, (ROWS * kD + ROWS + rl + ql) * 4, 0, kSys));
                const float m0 = c0 ? m[g] : mo, m1 = c0 ? mo : m[g];
                const float lt0 = c0 ? lt[g] : lto, lt1 = c0 ? lto : lt[g];
                const float mg = fmax_nan(m0, m1);
                const float w0 = m0 == -INFINITY ? 0.f : exp2f_fast(m0 - mg);
                const float w1 = m1 == -INFINITY ? 0.f : exp2f_fast(m1 - mg);
                const float inv = 1.f / (w0 * lt0 + w1 * lt1);
                const float a0 = w0 * inv, a1 = w1 * inv;
                if constexpr (WLSE) {
                    const float lo = __uint_as_float(
                        __builtin_amdgcn_raw_buffer_load_b32(rother, (ROWS * kD + 2 * ROWS + rl + ql) * 4, 0, kSys));
                    const float l0 = c0 ? l[g] : lo, l1 = c0 ? lo : l[g];
                    const int myq = q0 + rl + ql;
                    if (h == 0 && myq < Nq) LSE[(size_t)bh * Nq + myq] = (mg + log2f_fast(w0 * l0 + w1 * l1)) * kLn2;
                }
                if (QG > 1) stage_o(g);  // (with one group the stage still holds it)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int row = 4 * j + (lane >> 4);
                    const float a0r = __shfl(a0, row), a1r = __shfl(a1, row);
                    const int q = q0 + rl + row;
#pragma unroll
                    for (int hc = 0; hc < D / 64; ++hc) {
                        const int col = 64 * hc + 4 * (lane & 15);
                        const f32x4 own =
                            *reinterpret_cast<const f32x4 *>(stage + row * kD + (col ^ (4 * (row & 7))));
                        const f32x4 oth = __builtin_bit_cast(
                            f32x4, __builtin_amdgcn_raw_buffer_load_b128(rother, ((rl + row) * kD + col) * 4, 0, kSys));
                        const f32x4 o0 = c0 ? own : oth, o1 = c0 ? oth : own;
                        const f32x4 o = a0r * o0 + a1r * o1;
                        if (q < Nq)
                            *reinterpret_cast<u32x2 *>(O + ((size_t)bh * Nq + q) * kD + col) =
                                u32x2{pack2<DT>(o[0], o[1]), pack2<DT>(o[2], o[3])};
                    }
                }
            }
            return;
        }
        const size_t nch = gridDim.y;
#pragma unroll
        for (int g = 0; g < QG; ++g) {
            const int myq = qw + 32 * g + ql;
            stage_o(g);
            if (myq < Nq && h == 0) {
                const size_t pidx = ((size_t)bh * Nq + myq) * nch + blockIdx.y;
                m_part[pidx] = m[g] == -INFINITY ? -INFINITY : m[g] * kLn2;  // natural-log units
                l_part[pidx] = lt[g];
                if constexpr (WLSE) l2_part[pidx] = l[g];
            }
            // lane i of each 16-lane group writes 16 bytes of row 4j + lane/16,
            // columns 64 hc + 4 (lane % 16)
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int hc = 0; hc < D / 64; ++hc) {
                    const int row = 4 * j + (lane >> 4);
                    const int col = 64 * hc + 4 * (lane & 15);
                    const int q = qw + 32 * g + row;
                    const f32x4 val =
                        *reinterpret_cast<const f32x4 *>(stage + row * kD + (col ^ (4 * (row & 7))));
                    if (q < Nq)
                        *reinterpret_cast<f32x4 *>(o_part + (((size_t)bh * Nq + q) * nch + blockIdx.y) * kD +
                                                   col) = val;
                }
        }
        return;
    }
#pragma unroll
    for (int g = 0; g < QG; ++g) {
        const int myq = qw + 32 * g + ql;
        if (myq < Nq) {
            const float inv = 1.f / lt[g];
            uint16_t *orow = O + ((size_t)bh * Nq + myq) * kD;
#pragma unroll
            for (int dt = 0; dt < NT; ++dt)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int d = 32 * dt + 8 * g4 + 4 * h;
                    const int r = 4 * g4;
                    u32x2 w;
                    w[0] = pack2<DT>(oacc[g][dt][r] * inv, oacc[g][dt][r + 1] * inv);
                    w[1] = pack2<DT>(oacc[g][dt][r + 2] * inv, oacc[g][dt][r + 3] * inv);
                    *reinterpret_cast<u32x2 *>(orow + d) = w;
                }
            if constexpr (WLSE) {
                if (h == 0) LSE[(size_t)bh * Nq + myq] = (m[g] + log2f_fast(l[g])) * kLn2;
            }
        }
    }
}


// ---------------------------------------------------------------------------
// The same forward (keys not split) on v_mfma_f32_16x16x32_{f16,bf16}, whose
// 16-row tiles let a wave own QB blocks of 16 query rows.  With QB = 1 a
// shape whose 32-row waves would fill at most half of the wave slots gets
// twice the waves (16 rows each), with no split of the keys and no merge;
// every wave still walks all of its rows' keys.  Per 32-key tile and wave,
// with kb in {0, 1} the 16-key blocks, qb < QB the 16-query blocks and dc the
// 32-wide chunks of D:
//     S^T[kb][qb] = sum_dc K[16 keys of kb][32 d of dc] Q^T[32 d][16 queries of qb]
//     O^T[db][qb] += V^T[16 d of db][32 keys] P^T[32 keys][16 queries of qb]
// Register layouts (16x16x32 MFMA: A lane l holds row l%16, contraction
// slots 8(l/16)..+7; B lane l column l%16, the same slots; accumulator lane l
// register r holds row 4(l/16) + r, column l%16), with g = l/16, c = l%16:
//   * S^T[kb][qb] register r: key 16kb + 4g + r, query 16qb + c.  A lane thus
//     holds 8 scores of each of its QB queries; a query's 32 scores of the
//     tile lie in the four lanes c, c+16, c+32, c+48.
//   * P^T for query block qb is the B operand as it stands: contraction slot
//     j of lane (g, c) is key 16(j/4) + 4g + j%4, i.e. registers (kb, r) =
//     (j/4, j%4) of S^T[kb][qb], packed in pairs.
//   * V^T[db] pairs the same slots: two transposed LDS reads, keys 4g..4g+3
//     and 16+4g..16+4g+3, column 16db + c.
//   * O^T[db][qb] register r: d = 16db + 4g + r, query 16qb + c.
template <int DT>
struct Mfma16T;
template <>
struct Mfma16T<1> {
    static __device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                      __builtin_bit_cast(half8, b), c, 0, 0, 0);
    }
};
template <>
struct Mfma16T<2> {
    static __device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

template <int D, int DT, bool CAUSAL, bool WLSE, int QB>
__global__ __launch_bounds__(kWaves * 64, D == 64 ? 3 : 2) void fwd_mfma16_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, uint16_t *__restrict__ O, float *__restrict__ LSE,
    int Nq, int Nk, float scale_log2, int n_qtiles, int n_tiles, int snake) {
    static_assert(D == 64 || D == 128, "head dimension");
    constexpr int kD = D;
    constexpr int NDC = D / 32;                     // 32-wide contraction chunks of S^T
    constexpr int NDB = D / 16;                     // 16-row blocks of O^T
    constexpr int CPR = D / 8;                      // 16-byte chunks per LDS row
    constexpr int UPL = kBC * CPR / (kWaves * 64);  // 16-byte DMA units per lane per block
    constexpr int ROWS = kWaves * 16 * QB;          // query rows per workgroup
    // LDS: as in fwd_mfma_kernel (K buffers one 32-key tile ahead of V's).
    __shared__ __attribute__((aligned(16))) uint16_t sK0[kBC * kD];
    __shared__ __attribute__((aligned(16))) uint16_t sK1[kBC * kD];
    __shared__ __attribute__((aligned(16))) uint16_t sV0[kBC * kD];
    __shared__ __attribute__((aligned(16))) uint16_t sV1[kBC * kD];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;
    const int c = lane & 15;

    // Tile order: as in fwd_mfma_kernel.
    int bh, qt;
    if (CAUSAL && snake > 0) {
        const int per_xcd = n_tiles >> 3, hpx = per_xcd / n_qtiles;
        const int xcd = blockIdx.x & 7, pos = blockIdx.x >> 3;
        const int r = pos / snake, i = pos - r * snake;
        const int cnt = min(snake, per_xcd - r * snake);
        const int k = r * snake + ((r & 1) ? cnt - 1 - i : i);
        qt = n_qtiles - 1 - k / hpx;
        bh = xcd * hpx + k % hpx;
    } else if (CAUSAL) {
        const int n_bh = n_tiles / n_qtiles;
        const int rank = (int)blockIdx.x / n_bh;
        qt = n_qtiles - 1 - rank;
        bh = (int)blockIdx.x - rank * n_bh;
    } else {
        int wg = blockIdx.x;
        if ((n_tiles & 7) == 0) wg = (wg & 7) * (n_tiles >> 3) + (wg >> 3);
        bh = wg / n_qtiles;
        qt = wg - bh * n_qtiles;
    }
    const int q0 = qt * ROWS;
    const int qw = q0 + wave * 16 * QB;  // first row of this wave

    const uint16_t *Qh = Q + (size_t)bh * Nq * kD;
    const uint16_t *Kh = K + (size_t)bh * Nk * kD;
    const uint16_t *Vh = V + (size_t)bh * Nk * kD;
    const auto rq = make_rsrc(Qh, (uint32_t)Nq * kD * 2);
    const auto rk = make_rsrc(Kh, (uint32_t)Nk * kD * 2);
    const auto rv = make_rsrc(Vh, (uint32_t)Nk * kD * 2);

    // Scale sign and zero: as in fwd_mfma_kernel.
    const uint32_t qflip = scale_log2 < 0.f ? 0x80008000u : 0u;
    const uint32_t qkeep = scale_log2 == 0.f ? 0u : 0xFFFFFFFFu;
    scale_log2 = scale_log2 == 0.f ? 1.f : fabsf(scale_log2);

    // B operand of S^T for query block qb, chunk dc: slot j of lane (g, c) is
    // Q[qw + 16qb + c][32dc + 8g + j].
    u32x4 qf[QB][NDC];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc)
            qf[qb][dc] = load16(rq, (uint32_t)(((qw + 16 * qb + c) * kD + 32 * dc + 8 * g) * 2));

    const int kend = CAUSAL ? min(Nk, q0 + ROWS) : Nk;
    const int nblk = (kend + kBC - 1) / kBC;
    const int t_last = CAUSAL ? min((kend + 31) / 32 - 1, (qw + 16 * QB - 1) / 32) : 2 * nblk - 1;

    if (Nk % kBC != 0) {
        u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < UPL; ++i) {
            reinterpret_cast<u32x4 *>(sV0)[tid + 256 * i] = z;
            reinterpret_cast<u32x4 *>(sV1)[tid + 256 * i] = z;
        }
        __syncthreads();
    }

    // Block copies: as in fwd_mfma_kernel.
    auto dma = [&](const __amdgpu_buffer_rsrc_t &r, uint16_t *dst, int k0, bool r_is_k) {
#pragma unroll
        for (int i = 0; i < UPL; ++i) {
            const int unit = (UPL * wave + i) * 64 + lane;
            const int row = unit / CPR;
            const int ch = (unit % CPR) ^ (r_is_k ? kswz<D>(row) : vswz<D>(row));
            const int key = k0 + row;
            const uint32_t off = key < 0 ? 0xFFFFFFF0u : (uint32_t)((key * kD + ch * 8) * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst + (UPL * wave + i) * 512), 16,
                                                     off, 0, 0, 0);
        }
    };
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    auto dma_at = [&](const uint16_t *X, uint16_t *dst, int k0, bool r_is_k) {
        const int kb = k0 < Nk ? k0 : Nk;
        const auto r = make_rsrc(X + (size_t)kb * kD, (uint32_t)(Nk - kb) * kD * 2);
#pragma unroll
        for (int i = 0; i < UPL; ++i) {
            const int unit = (UPL * wave + i) * 64 + lane;
            const int row = unit / CPR;
            const int ch = (unit % CPR) ^ (r_is_k ? kswz<D>(row) : vswz<D>(row));
            const uint32_t off = (uint32_t)((row * kD + ch * 8) * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst + (UPL * wave_s + i) * 512), 16,
                                                     off, 0, 0, 0);
        }
    };

    // LDS offsets relative to a tile's first row (both halves of a 64-row
    // buffer share the swizzle).  K: row 16kb + c, chunk 4dc + g.  V (the
    // transposed read, 4 rows x 16 columns per 16-lane group): lane c points at
    // row 4g + c/4 + 16u and columns 16db + 4(c%4) .. +3, and receives column
    // 16db + c of those 4 rows.
    int kofs[2][NDC], vofs[NDB][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) {
            const int key = 16 * kb + c;
            kofs[kb][dc] = key * kD + (((4 * dc + g) ^ kswz<D>(key)) << 3);
        }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int key = 4 * g + (c >> 2) + 16 * u;
            const int d = 16 * db + 4 * (c & 3);
            vofs[db][u] = key * kD + (((d >> 3) ^ vswz<D>(key)) << 3) + (d & 7);
        }

    float m[QB], mu[QB], l[QB], lt[QB];  // per query block: max used for the exponentials
                                         // (base 2), that max or 0 while the row has none,
                                         // this lane's shares of the denominators (f32 P,
                                         // rounded P)
    // Wave-uniform: some lane's row has no max yet (every tile then takes the max).
    bool no_max = true;
    const uint32_t ones = DT == 1 ? 0x3C003C00u : 0x3F803F80u;
    f32x4 oacc[NDB][QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m[qb] = -INFINITY;
        mu[qb] = 0.f;
        l[qb] = lt[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // One 32-key tile t; scur holds S^T of tile t ([kb][qb]), kn points at the
    // LDS rows of tile t+1's keys and vt at those of tile t's values.  With
    // NEXT the scores of tile t+1 go to snext, issued among this tile's
    // exponentials.
    auto tile = [&](const int t, const uint16_t *kn, const uint16_t *vt, f32x4 (*scur)[QB],
                    f32x4 (*snext)[QB], auto next_tag) {
        constexpr bool NEXT = decltype(next_tag)::value;
        const int k0 = 32 * t;
        u32x4 kf[2][NDC];
        if constexpr (NEXT) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int dc = 0; dc < NDC; ++dc)
                    kf[kb][dc] = *reinterpret_cast<const u32x4 *>(&kn[kofs[kb][dc]]);
        }
        u32x4 vf[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vt + vofs[db][0]));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vt + vofs[db][1]));
            const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
            const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
            vf[db] = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
        }

        const bool need_mask = (k0 + 32 > Nk) || (CAUSAL && k0 + 31 > qw);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int key = k0 + 16 * kb + 4 * g + r;
                        bool ok = key < Nk;
                        if (CAUSAL) ok = ok && key <= qw + 16 * qb + c;
                        if (!ok) scur[kb][qb][r] = -INFINITY;
                    }
        }
        // P of query block qb, packed as its B operand (pk[qb][2kb + r/2]),
        // with the row sums of the rounded P (lp) and of the f32 P (ps).
        u32x4 pk[QB];
        float ps[QB], lp[QB];
        auto exps = [&](int qb, float m_use, bool with_next) __attribute__((always_inline)) {
            ps[qb] = 0.f;
            float lp0 = 0.f, lp1 = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const float x0 = __builtin_fmaf(scur[kb][qb][2 * h2], scale_log2, -m_use);
                    const float x1 = __builtin_fmaf(scur[kb][qb][2 * h2 + 1], scale_log2, -m_use);
                    const float p0 = exp2f_fast(x0);
                    const float p1 = exp2f_fast(x1);
                    const uint32_t w = pack2<DT>(p0, p1);
                    pk[qb][2 * kb + h2] = w;
                    if constexpr (WLSE) ps[qb] += p0 + p1;
                    if (h2 == 0) lp0 = dot2<DT>(w, ones, lp0); else lp1 = dot2<DT>(w, ones, lp1);
                    if constexpr (NEXT) {
                        // the next tile's score block (kb, qb), among this block's exponentials
                        if (with_next && h2 == 0) {
#pragma unroll
                            for (int dc = 0; dc < NDC; ++dc)
                                snext[kb][qb] = Mfma16T<DT>::mma(kf[kb][dc], qf[qb][dc],
                                                               dc == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : snext[kb][qb]);
                        }
                    }
                }
            lp[qb] = lp0 + lp1;
        };
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) exps(qb, mu[qb], true);
        // Conditional rescaling: as in fwd_mfma_kernel, one test for all query
        // blocks (taking the max of a block whose P stayed under the cap is
        // also exact), the row max taken over the four lanes of each query.
        float lpmax = lp[0];
#pragma unroll
        for (int qb = 1; qb < QB; ++qb) lpmax = fmaxf(lpmax, lp[qb]);
        if (no_max || __builtin_amdgcn_ballot_w64(lpmax > kLazyCap) != 0) {
            bool none = false;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                float mx = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, scur[kb][qb][r]);
                mx = max_xor32(max_xor16(mx)) * scale_log2;
                const float m_new = fmaxf(m[qb], mx);
                mu[qb] = m_new == -INFINITY ? 0.f : m_new;
                const float corr = exp2f_fast(m[qb] - mu[qb]);
                l[qb] *= corr;
                lt[qb] *= corr;
#pragma unroll
                for (int db = 0; db < NDB; ++db) oacc[db][qb] *= corr;
                m[qb] = m_new;
                none = none || m_new == -INFINITY;
                exps(qb, mu[qb], false);
            }
            no_max = __builtin_amdgcn_ballot_w64(none) != 0;
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[db][qb] = Mfma16T<DT>::mma(vf[db], pk[qb], oacc[db][qb]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            lt[qb] += lp[qb];
            if constexpr (WLSE) l[qb] += ps[qb];
        }
    };

    auto run_tile = [&](const int t, const uint16_t *kn, const uint16_t *vt, f32x4 (*scur)[QB],
                        f32x4 (*snext)[QB]) {
        if constexpr (CAUSAL) {
            if (t > t_last) return;
            if (t + 1 <= t_last)
                tile(t, kn, vt, scur, snext, std::true_type{});
            else
                tile(t, kn, vt, scur, snext, std::false_type{});
        } else {
            tile(t, kn, vt, scur, snext, std::true_type{});
        }
    };

    auto block = [&](int b, const uint16_t *kc, uint16_t *kd, const uint16_t *vc, uint16_t *vd,
                     f32x4 (*sa)[QB], f32x4 (*sb)[QB]) {
        if (b + 1 < nblk) {
            dma_at(Vh, vd, (b + 1) * kBC, false);
            dma_at(Kh, kd, (b + 1) * kBC + 32, true);
        }
        run_tile(2 * b, kc, vc, sa, sb);
        run_tile(2 * b + 1, kc + 32 * kD, vc + 32 * kD, sb, sa);
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
    };

    if (nblk > 0) {
        dma(rv, sV0, 0, false);
        dma(rk, sK0, 32, true);
        dma(rk, sK1, -32, true);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int dc = 0; dc < NDC; ++dc) qf[qb][dc] = (qf[qb][dc] ^ qflip) & qkeep;
        f32x4 sa[2][QB], sb[2][QB];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int dc = 0; dc < NDC; ++dc) {
                    const u32x4 a = *reinterpret_cast<const u32x4 *>(&sK1[32 * kD + kofs[kb][dc]]);
                    sa[kb][qb] = Mfma16T<DT>::mma(a, qf[qb][dc], dc == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sa[kb][qb]);
                }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        for (int b = 0; b < nblk; b += 2) {
            block(b, sK0, sK1, sV0, sV1, sa, sb);
            if (b + 1 < nblk) block(b + 1, sK1, sK0, sV1, sV0, sa, sb);
        }
    }

    // Each query's sums over its four lanes.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        lt[qb] += __shfl_xor(lt[qb], 16);
        lt[qb] += __shfl_xor(lt[qb], 32);
        if constexpr (WLSE) {
            l[qb] += __shfl_xor(l[qb], 16);
            l[qb] += __shfl_xor(l[qb], 32);
        }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int myq = qw + 16 * qb + c;
        if (myq < Nq) {
            const float inv = 1.f / lt[qb];
            uint16_t *orow = O + ((size_t)bh * Nq + myq) * kD;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                u32x2 w;
                w[0] = pack2<DT>(oacc[db][qb][0] * inv, oacc[db][qb][1] * inv);
                w[1] = pack2<DT>(oacc[db][qb][2] * inv, oacc[db][qb][3] * inv);
                *reinterpret_cast<u32x2 *>(orow + 16 * db + 4 * g) = w;
            }
            if constexpr (WLSE) {
                if (g == 0) LSE[(size_t)bh * Nq + myq] = (m[qb] + log2f_fast(l[qb])) * kLn2;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Few query rows: one workgroup per 32 query rows whose W waves each walk a
// contiguous slice of the keys, then merge their W partial states through LDS
// with the (m, l) monoid ("Flash Attention", section Deriving the online
// softmax: any grouping of the keys gives the same result).  This is the
// key split of "Flash decoding" done inside one workgroup, so a shape with
// too few query tiles to fill the device needs neither a workspace for
// partials nor a second launch to combine them.
//
// Per wave and 32-key tile the arithmetic is that of fwd_mfma_kernel (S^T =
// K Q^T with the next tile's scores issued during this tile's exponentials,
// conditional rescaling, P rounded to the input dtype, O^T += V^T P^T).  K
// goes straight from global memory into the MFMA A-operand registers (16
// contiguous bytes per lane); V goes through the wave's own LDS double buffer
// (a DMA per tile, swizzled as in fwd_mfma_kernel) for the transposed read;
// K of tile t+2 and V of tile t+1 are in flight while tile t is computed.
// After the walk the same LDS holds each wave's unnormalised O (32 x D floats).
template <int D, int DT, bool CAUSAL, bool WLSE, int W>
__global__ __launch_bounds__(W * 64, 1) void fwd_rows_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, uint16_t *__restrict__ O, float *__restrict__ LSE, int Nq,
    int Nk, float scale_log2, int n_qtiles) {
    static_assert(D == 64, "head dimension");
    constexpr int kD = D;
    constexpr int NC = D / 16;            // 16-wide contraction chunks of S^T = K Q^T
    constexpr int NT = D / 32;            // 32-column tiles of O^T
    constexpr int CPR = D / 8;            // 16-byte chunks per row
    constexpr int UPW = 32 * CPR / 64;    // 16-byte DMA units per lane per V tile
    constexpr int TILE = 32 * D;          // 16-bit elements of one V tile
    __shared__ __attribute__((aligned(16))) uint16_t sV[W * 2 * TILE];
    __shared__ float s_m[W][32], s_lt[W][32], s_l[W][32];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5;
    const int ql = lane & 31;

    // b*h varies fastest; causal: the longest tiles first
    const int n_bh = gridDim.x / n_qtiles;
    int qt = blockIdx.x / n_bh;
    const int bh = blockIdx.x - qt * n_bh;
    if (CAUSAL) qt = n_qtiles - 1 - qt;
    const int q0 = qt * 32;

    const uint16_t *Qh = Q + (size_t)bh * Nq * kD;
    const uint16_t *Kh = K + (size_t)bh * Nk * kD;
    const uint16_t *Vh = V + (size_t)bh * Nk * kD;
    const auto rq = make_rsrc(Qh, (uint32_t)Nq * kD * 2);
    const auto rk = make_rsrc(Kh, (uint32_t)Nk * kD * 2);
    const auto rv = make_rsrc(Vh, (uint32_t)Nk * kD * 2);

    // a negative scale goes onto Q, a zero scale is Q = 0 with scale 1 (as in
    // fwd_mfma_kernel: maxima and masks are taken on unscaled scores)
    const uint32_t qflip = scale_log2 < 0.f ? 0x80008000u : 0u;
    const uint32_t qkeep = scale_log2 == 0.f ? 0u : 0xFFFFFFFFu;
    scale_log2 = scale_log2 == 0.f ? 1.f : fabsf(scale_log2);

    // B operand of S^T = K Q^T: chunk dc, slot (h, j) is Q[q0 + ql][16dc + 8h + j]
    u32x4 qf[NC];
#pragma unroll
    for (int dc = 0; dc < NC; ++dc)
        qf[dc] = (load16(rq, (uint32_t)(((q0 + ql) * kD + 16 * dc + 8 * h) * 2)) ^ qflip) & qkeep;

    // this wave's 32-key tiles [t0, t1)
    const int kend = CAUSAL ? min(Nk, q0 + 32) : Nk;
    const int ntiles = (kend + 31) / 32;
    const int per = (ntiles + W - 1) / W;
    const int t0 = min(ntiles, wave * per);
    const int t1 = min(ntiles, t0 + per);
    uint16_t *vbuf = sV + wave * 2 * TILE;

    // A operand of S^T = K Q^T for tile t: row ql is key 32t + ql, chunk dc
    // holds its columns 16dc + 8h .. + 8 (zeros past Nk)
    auto load_k = [&](int t, u32x4 (&kr)[NC]) __attribute__((always_inline)) {
#pragma unroll
        for (int dc = 0; dc < NC; ++dc)
            kr[dc] = load16(rk, (uint32_t)(((32 * t + ql) * kD + 16 * dc + 8 * h) * 2));
    };
    // V tile t -> LDS buffer t % 2: unit u of the tile holds chunk (u % CPR) ^
    // vswz(row) of row u / CPR (rows past Nk load zeros)
    auto dma_v = [&](int t) __attribute__((always_inline)) {
        uint16_t *dst = vbuf + (t & 1) * TILE;
#pragma unroll
        for (int i = 0; i < UPW; ++i) {
            const int unit = i * 64 + lane;
            const int row = unit / CPR;
            const int ch = (unit % CPR) ^ vswz<D>(row);
            const uint32_t off = (uint32_t)(((32 * t + row) * kD + ch * 8) * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(dst + i * 512), 16, off, 0, 0, 0);
        }
    };
    int vofs[NT][2];
    {
        const int i = lane & 15;
        const int kl = 4 * h + (i >> 2);
#pragma unroll
        for (int dt = 0; dt < NT; ++dt) {
            const int d = 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (i & 3);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int key = kl + 8 * u;
                vofs[dt][u] = key * kD + (((d >> 3) ^ vswz<D>(key)) << 3) + (d & 7);
            }
        }
    }

    float m = -INFINITY, l = 0.f, lt = 0.f;
    const uint32_t ones = DT == 1 ? 0x3C003C00u : 0x3F803F80u;
    f32x16 oacc[NT];
#pragma unroll
    for (int dt = 0; dt < NT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;

    // Tile t: scur holds S^T of tile t, kn the K operand of tile t+1 (NEXT);
    // kld receives that of tile t+2.
    auto tile = [&](const int t, const u32x4 (&kn)[NC], u32x4 (&kld)[NC], f32x16 &scur,
                    f32x16 &snext, auto next_tag) __attribute__((always_inline)) {
        constexpr bool NEXT = decltype(next_tag)::value;
        // V of tile t has landed, K of tile t+1 is in registers, and every LDS
        // read of tile t-1 is done (its buffer takes tile t+1's V next)
        __builtin_amdgcn_s_waitcnt(0);
        if (t + 2 < t1) load_k(t + 2, kld);
        if constexpr (NEXT) dma_v(t + 1);
        const uint16_t *vt = vbuf + (t & 1) * TILE;
        u32x4 vf[2][NT];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int dt = 0; dt < NT; ++dt) {
                const uint16_t *src = vt + 16 * c * kD;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(src + vofs[dt][0]));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(src + vofs[dt][1]));
                const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
                const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
                vf[c][dt] = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
            }
        const int k0 = 32 * t;
        if ((k0 + 32 > Nk) || (CAUSAL && k0 + 31 > q0)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + 8 * (r >> 2) + 4 * h + (r & 3);
                bool ok = key < Nk;
                if (CAUSAL) ok = ok && key <= q0 + ql;
                if (!ok) scur[r] = -INFINITY;
            }
        }
        u32x4 pk[2];
        float ps[2], lp[2];
        auto exps = [&](float m_use, bool with_next) __attribute__((always_inline)) {
            ps[0] = ps[1] = lp[0] = lp[1] = 0.f;
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 8 * c + 2 * j;
                    const float p0 = exp2f_fast(__builtin_fmaf(scur[r], scale_log2, -m_use));
                    const float p1 = exp2f_fast(__builtin_fmaf(scur[r + 1], scale_log2, -m_use));
                    const uint32_t w = pack2<DT>(p0, p1);
                    pk[c][j] = w;
                    if constexpr (WLSE) ps[j & 1] += p0 + p1;
                    lp[j & 1] = dot2<DT>(w, ones, lp[j & 1]);
                    if constexpr (NEXT) {
                        if (with_next && c == 0)
                            snext = MfmaT<DT>::mma(kn[j], qf[j], j == 0 ? f32x16{} : snext);
                    }
                }
        };
        // conditional rescaling, as in fwd_mfma_kernel
        exps(m == -INFINITY ? 0.f : m, true);
        if (__builtin_amdgcn_ballot_w64(m == -INFINITY || lp[0] + lp[1] > kLazyCap) != 0) {
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, scur[r]);
            mx = max_halves(mx) * scale_log2;
            const float m_new = fmaxf(m, mx);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float corr = exp2f_fast(m - m_use);
            l *= corr;
            lt *= corr;
#pragma unroll
            for (int dt = 0; dt < NT; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[dt][i] *= corr;
            m = m_new;
            exps(m_use, false);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int dt = 0; dt < NT; ++dt) oacc[dt] = MfmaT<DT>::mma(vf[c][dt], pk[c], oacc[dt]);
        lt += lp[0] + lp[1];
        if constexpr (WLSE) l += ps[0] + ps[1];
    };
    auto run_tile = [&](const int t, const u32x4 (&kn)[NC], u32x4 (&kld)[NC], f32x16 &scur,
                        f32x16 &snext) __attribute__((always_inline)) {
        if (t + 1 < t1)
            tile(t, kn, kld, scur, snext, std::true_type{});
        else
            tile(t, kn, kld, scur, snext, std::false_type{});
    };

    if (t0 < t1) {  // (wave-uniform)
        u32x4 ka[NC], kb[NC];
        load_k(t0, ka);
        dma_v(t0);
        load_k(t0 + 1, kb);  // (in-range rows or zeros when t0 + 1 >= t1; then unused)
        f32x16 sa, sb;
#pragma unroll
        for (int dc = 0; dc < NC; ++dc) sa = MfmaT<DT>::mma(ka[dc], qf[dc], dc == 0 ? f32x16{} : sa);
        for (int t = t0; t < t1; t += 2) {
            run_tile(t, kb, ka, sa, sb);
            if (t + 1 < t1) run_tile(t + 1, ka, kb, sb, sa);
        }
    }

    // Merge.  oacc[dt][r] = O[q0 + ql][32dt + 8(r/4) + 4h + r%4] (unnormalised,
    // base-2 max m); each lane holds half of the row's sums.
    lt += __shfl_xor(lt, 32);
    if constexpr (WLSE) l += __shfl_xor(l, 32);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // every wave is done with its V buffers
    float *so = reinterpret_cast<float *>(sV) + wave * 32 * kD;
#pragma unroll
    for (int dt = 0; dt < NT; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int r = 4 * g4;
            *reinterpret_cast<f32x4 *>(so + ql * kD + ((32 * dt + 8 * g4 + 4 * h) ^ (4 * (ql & 7)))) =
                f32x4{oacc[dt][r], oacc[dt][r + 1], oacc[dt][r + 2], oacc[dt][r + 3]};
        }
    if (h == 0) {
        s_m[wave][ql] = m;
        s_lt[wave][ql] = lt;
        s_l[wave][ql] = l;
    }
    __syncthreads();
    // one thread per row: the row's max, each wave's weight 2^(m_w - m) (into
    // s_m), 1 / sum of the rounded-P denominators (into s_lt[0]) and the LSE
    if (threadIdx.x < 32) {
        const int row = threadIdx.x;
        float mg = -INFINITY;
#pragma unroll
        for (int w = 0; w < W; ++w) mg = fmaxf(mg, s_m[w][row]);
        float ltg = 0.f, lg = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const float mw = s_m[w][row];
            const float a = mw == -INFINITY ? 0.f : exp2f_fast(mw - mg);
            s_m[w][row] = a;
            ltg += a * s_lt[w][row];
            if constexpr (WLSE) lg += a * s_l[w][row];
        }
        s_lt[0][row] = 1.f / ltg;
        if constexpr (WLSE) {
            if (q0 + row < Nq) LSE[(size_t)bh * Nq + q0 + row] = (mg + log2f_fast(lg)) * kLn2;
        }
    }
    __syncthreads();
    // four consecutive output columns per thread and pass
    const float *sall = reinterpret_cast<const float *>(sV);
    for (int e = 4 * (int)threadIdx.x; e < 32 * kD; e += 4 * W * 64) {
        const int row = e / kD, col = e % kD;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(sall + (w * 32 + row) * kD +
                                                             (col ^ (4 * (row & 7))));
            acc += s_m[w][row] * v;
        }
        const float inv = s_lt[0][row];
        if (q0 + row < Nq) {
            u32x2 out;
            out[0] = pack2<DT>(acc[0] * inv, acc[1] * inv);
            out[1] = pack2<DT>(acc[2] * inv, acc[3] * inv);
            *reinterpret_cast<u32x2 *>(O + ((size_t)bh * Nq + q0 + row) * kD + col) = out;
        }
    }
}

// Waves of fwd_rows_kernel (two per SIMD), each on its own slice of the keys.
// The kernel runs at D = 64: at D = 128 its ring of operands does not fit two
// waves' registers, and the key split across workgroups measured faster there.
#ifndef FA2_ROWS_WAVES
#define FA2_ROWS_WAVES 8  // waves of fwd_rows_kernel (splitting the keys of 32 query rows)
#endif
constexpr int kRowsWaves = FA2_ROWS_WAVES;

struct Plan {
    int qg, n_qtiles, n_tiles, chunks;
    bool rows;  // few query tiles: fwd_rows_kernel (32-row workgroups, keys split across waves)
    bool q16;   // 16-row waves: fwd_mfma16_kernel with one query block per wave (64-row tiles)
};

#ifndef FA2_MFMA_SPLIT_WGS
#define FA2_MFMA_SPLIT_WGS 2  // target workgroups per compute unit when splitting keys
#endif
#ifndef FA2_MFMA_SPLIT_BELOW
#define FA2_MFMA_SPLIT_BELOW 8  // split only with at most num_cus / this many query tiles
#endif
#ifndef FA2_MFMA_QG2
#define FA2_MFMA_QG2 1  // 1: 64 query rows per wave when the tiles fill the device twice over; 2: always
#endif
#ifndef FA2_MFMA_SNAKE
#define FA2_MFMA_SNAKE 1  // causal tiles in one round: deal them to CUs in a snake by length
#endif
#ifndef FA2_MFMA_ROWS
#define FA2_MFMA_ROWS 1  // few query tiles: one launch of fwd_rows_kernel instead of split + combine
#endif
#ifndef FA2_MFMA_ROWS_MAX_NK
#define FA2_MFMA_ROWS_MAX_NK 2048  // ... only when the keys are at most this long (with longer
                                   // keys the key split across workgroups measured faster)
#endif
#ifndef FA2_MFMA_SPLIT_LONG
#define FA2_MFMA_SPLIT_LONG 32  // also split when the tiles fill at most a quarter of the slots
                                // and the keys span at least this many 64-key blocks (0: never)
#endif
#ifndef FA2_MFMA_PAIR
#define FA2_MFMA_PAIR 1  // more shapes split in two, merged in the kernel (0: off)
#endif
#ifndef FA2_MFMA_Q16
#define FA2_MFMA_Q16 1  // 16-row waves on 16x16x32 MFMAs when 32-row waves fill at most half the slots (D = 64)
#endif
#ifndef FA2_MFMA_Q16_D128
#define FA2_MFMA_Q16_D128 1  // the same at D = 128 (two workgroups per CU), causal shapes
#endif
#ifndef FA2_MFMA_SPLIT_LONG_HALF
#define FA2_MFMA_SPLIT_LONG_HALF 64  // ... or at most half of the slots and at least this many
                                      // blocks (0: never)
#endif

// Query groups per wave: 64-row waves when the 256-row tiles make whole
// rounds of two per compute unit.  Keys: split the keys of each query tile
// when the query tiles fill at most an eighth of the compute units (with
// more, writing and merging the partials costs more than the idle units),
// into at most one chunk per two key blocks; with more tiles, see below.
Plan plan(int B, int H, int Nq, int Nk, int D, int causal, int num_cus) {
    Plan p;
    p.qg = 1;
    if (FA2_MFMA_QG2 && D == 64) {
        const long long nt2 = (long long)((Nq + 2 * kBR - 1) / (2 * kBR)) * B * H;
        if (FA2_MFMA_QG2 == 2 || (nt2 >= 2LL * num_cus && nt2 % (2LL * num_cus) == 0)) p.qg = 2;
    }
    p.n_qtiles = (Nq + kBR * p.qg - 1) / (kBR * p.qg);
    const long long nt = (long long)p.n_qtiles * B * H;
    p.n_tiles = nt > 0x7FFFFFFF ? -1 : (int)nt;
    p.chunks = 1;
    p.rows = false;
    p.q16 = false;
    const long long nblk = (Nk + kBC - 1) / kBC;
    const long long nt32 = (long long)((Nq + 31) / 32) * B * H;
    if (FA2_MFMA_ROWS && D == 64 && nt > 0 && nt * FA2_MFMA_SPLIT_BELOW <= num_cus &&
        Nk <= FA2_MFMA_ROWS_MAX_NK && nt32 <= 0x7FFFFFFF) {
        p.rows = true;
    } else if (nt > 0 && nt * FA2_MFMA_SPLIT_BELOW <= num_cus) {
        long long c = ((long long)FA2_MFMA_SPLIT_WGS * num_cus + nt - 1) / nt;
        c = std::min<long long>(c, std::max<long long>(1, nblk / 2));
        p.chunks = (int)std::min<long long>(c, 32);
    } else if (FA2_MFMA_SPLIT_LONG > 0 && nt > 0 && nblk >= FA2_MFMA_SPLIT_LONG) {
        // Long keys with the tiles filling at most a quarter of the resident
        // workgroup slots: cut the keys so the chunks fill the slots (the
        // partials then cost little next to the work of each chunk).  At half
        // the slots only with long keys: B4 H12 with 1024 queries split in
        // two measured 39.2 -> 43.3 us at 2048 keys, 77.0 -> 72.7 us at 4096
        // (bf16 with LSE 77.2 -> 70.9), 140.1 -> 125.6 us at 8192.
        const long long slots = (long long)num_cus * (p.qg == 1 && D == 64 ? 3 : 2);
        if (4 * nt <= slots ||
            (FA2_MFMA_SPLIT_LONG_HALF > 0 && nblk >= FA2_MFMA_SPLIT_LONG_HALF && 2 * nt <= slots)) {
            const long long c = std::min<long long>(slots / nt, nblk / 16);
            p.chunks = (int)std::max<long long>(1, std::min<long long>(c, 32));
        }
    }
    if (FA2_MFMA_PAIR && p.chunks == 1 && !p.rows && nt > 0) {
        // Two chunks, merged in the kernel by the tile's second workgroup
        // (no combine launch, so the split pays at shorter keys): when the
        // tiles fill at most an eighth of the workgroup slots (keys of 16
        // blocks or more), and at D = 64 when they fill at most half of the
        // slots with keys of 32 blocks or more, if the tiles are causal (the
        // halves of the longest tiles set the time) or if the halves lower
        // the most tiles any compute unit holds (384 tiles: two on some CUs
        // unsplit, three halves on every CU split; 256 tiles: one either way).
        // Measured: B1 H8 1024^2 f16 14.4 -> 13.5 us, causal 17.7 -> 14.7,
        // D = 128 21.5 -> 17.7; B2 H12 2048^2 causal 34.5 -> 29.9, unmasked
        // 40.2 -> 39.3; B4 H12 1024 x 3000 56.9 -> 52.4; against B2 H8 2048^2
        // unmasked 27.2 -> 29.1 and B1 H12 2048^2 D128 38.1 -> 39.8 split.
        const long long slots = (long long)num_cus * (p.qg == 1 && D == 64 ? 3 : 2);
        const bool fewer = (2 * nt + num_cus - 1) / num_cus < 2 * ((nt + num_cus - 1) / num_cus);
        if ((8 * nt <= slots && nblk >= 16) ||
            (D == 64 && 2 * nt <= slots && nblk >= 32 && (causal || fewer)))
            p.chunks = 2;
    }
    const bool q16_fit = 2 * nt <= 3LL * num_cus &&
                         (D == 64 ? causal || 8 * nt >= 9LL * num_cus : FA2_MFMA_Q16_D128 && causal);
    if (FA2_MFMA_Q16 && p.qg == 1 && p.chunks == 1 && !p.rows && nt > 0 && q16_fit) {
        // The 128-row tiles fill at most half of the wave slots: 64-row tiles
        // of 16-row waves (fwd_mfma16_kernel, QB = 1) give twice the waves --
        // when causal (the shorter tiles also even out the mask's uneven
        // lengths), or when the doubled tiles fill at least three quarters of
        // the slots.  Measured (f16 unless noted): B4 H12 N1024 21.9 -> 20.2 us
        // (bf16 21.2 -> 19.6), causal 18.9 -> 16.1, B2 H12 N1024 causal 17.8 ->
        // 15.3, B8 H12 N512 causal 12.1 -> 10.1; against B4 H12 N512 9.38 ->
        // 9.48, B2 H12 N1000 bf16 14.3 -> 14.6, B2 H8 and B1 H16 N2048 24.8 ->
        // 25.4 with 16-row waves (half or two thirds of the slots filled).
        // At D = 128 (two workgroups per CU) only when causal: B2 H12 N1024
        // causal f16 24.8 -> 23.3 us, B4 H12 N512 causal bf16 15.5 -> 14.4,
        // B1 H16 N2048 causal 43.4 -> 41.3, B4 H12 N1024 causal 29.5 -> 27.4
        // (384 tiles); against B2 H16 N2048 causal 50.3 -> 54.2 (512 tiles)
        // and, unmasked, B2 H12 N1024 23.4 -> 26.9, B1 H12 N2048 37.3 -> 47.3.
        const long long nt64 = (long long)((Nq + 63) / 64) * B * H;
        if (nt64 <= 0x7FFFFFFF) {
            p.q16 = true;
            p.n_qtiles = (Nq + 63) / 64;
            p.n_tiles = (int)nt64;
        }
    }
    return p;
}

size_t part_bytes(const FwdArgs &a, int chunks) {
    return (size_t)a.B * a.H * a.Nq * chunks * (a.D + 3) * sizeof(float);
}

// Workspace of a two-chunk split merged in the kernel: one 8-byte handshake
// word per tile (the area padded to 256 bytes), then per tile and chunk a
// state block of rows * (D + 3) floats.
struct PairLayout {
    size_t tag_bytes, bytes;
    PairLayout(long long tiles, int rows, int D)
        : tag_bytes(((size_t)tiles * 8 + 255) & ~(size_t)255),
          bytes(tag_bytes + (size_t)tiles * 2 * rows * (D + 3) * sizeof(float)) {}
};

// CUs per XCD for the causal snake order (0: keep longest first): only when
// all tiles fit one round of workgroup slots and every XCD holds whole heads.
template <int D, int QG>
int snake_cus(const FwdArgs &a, const Plan &p) {
    if (!a.causal || FA2_MFMA_SNAKE == 0 || p.n_tiles % 8 != 0 || a.num_cus % 8 != 0) return 0;
    const int per_xcd = p.n_tiles / 8;
    const long long slots = (long long)a.num_cus * (QG == 1 && D == 64 ? 3 : 2);
    if (per_xcd % p.n_qtiles != 0 || p.n_tiles > slots) return 0;
    return a.num_cus / 8;
}

template <int D, int DT, bool CAUSAL, bool WLSE, int QG>
fa2_status launch_q(const FwdArgs &a, const Plan &p, hipStream_t st) {
    const uint16_t *q = (const uint16_t *)a.q, *k = (const uint16_t *)a.k, *v = (const uint16_t *)a.v;
    const float sl2 = a.scale * kLog2e;
    const PairLayout pair(p.n_tiles, kWaves * 32 * QG, D);
    if (p.chunks == 2 && a.ws && a.ws_bytes >= pair.bytes) {
        return launch(fwd_mfma_kernel<D, DT, CAUSAL, WLSE, true, QG>, dim3((unsigned)p.n_tiles, 2u),
                      dim3(kWaves * 64), st, q, k, v, (uint16_t *)a.o, a.lse,
                      (float *)((char *)a.ws + pair.tag_bytes), (float *)nullptr, (float *)nullptr,
                      (float *)nullptr, (unsigned long long *)a.ws, next_launch_tag(), a.Nq, a.Nk, sl2,
                      p.n_qtiles, p.n_tiles, 0);
    }
    if (p.chunks > 2 && a.ws && a.ws_bytes >= part_bytes(a, p.chunks)) {
        const size_t n = (size_t)a.B * a.H * a.Nq * p.chunks;
        float *o_part = (float *)a.ws;
        float *m_part = o_part + n * D;
        float *l_part = m_part + n;
        float *l2_part = l_part + n;
        fa2_status s = launch(fwd_mfma_kernel<D, DT, CAUSAL, WLSE, true, QG>,
                              dim3((unsigned)p.n_tiles, (unsigned)p.chunks), dim3(kWaves * 64), st,
                              q, k, v, (uint16_t *)a.o, a.lse, o_part, m_part, l_part, l2_part,
                              (unsigned long long *)nullptr, 0ull, a.Nq, a.Nk, sl2, p.n_qtiles,
                              p.n_tiles, 0);
        if (s != FA2_OK) return s;
        return launch_combine_rows(o_part, m_part, l_part, a.o, a.lse, (size_t)a.B * a.H * a.Nq, D,
                                   p.chunks, DT == 1 ? FA2_F16 : FA2_BF16, st,
                                   WLSE ? l2_part : nullptr);
    }
    if constexpr (QG == 1 && (D == 64 || FA2_MFMA_Q16_D128)) {
        if (p.q16)
            return launch(fwd_mfma16_kernel<D, DT, CAUSAL, WLSE, 1>, dim3((unsigned)p.n_tiles),
                          dim3(kWaves * 64), st, q, k, v, (uint16_t *)a.o, a.lse, a.Nq, a.Nk, sl2,
                          p.n_qtiles, p.n_tiles, snake_cus<D, QG>(a, p));
    }
    return launch(fwd_mfma_kernel<D, DT, CAUSAL, WLSE, false, QG>, dim3((unsigned)p.n_tiles),
                  dim3(kWaves * 64), st, q, k, v, (uint16_t *)a.o, a.lse, (float *)nullptr,
                  (float *)nullptr, (float *)nullptr, (float *)nullptr, (unsigned long long *)nullptr,
                  0ull, a.Nq, a.Nk, sl2, p.n_qtiles, p.n_tiles, snake_cus<D, QG>(a, p));
}

template <int D, int DT, bool CAUSAL, bool WLSE>
fa2_status launch_rows(const FwdArgs &a, hipStream_t st) {
    const int n_qtiles = (a.Nq + 31) / 32;
    const long long grid = (long long)n_qtiles * a.B * a.H;
    return launch(fwd_rows_kernel<D, DT, CAUSAL, WLSE, kRowsWaves>, dim3((unsigned)grid),
                  dim3(kRowsWaves * 64), st, (const uint16_t *)a.q, (const uint16_t *)a.k,
                  (const uint16_t *)a.v, (uint16_t *)a.o, a.lse, a.Nq, a.Nk, a.scale * kLog2e,
                  n_qtiles);
}

template <int D, int DT, bool CAUSAL, bool WLSE>
fa2_status launch_v(const FwdArgs &a, const Plan &p, hipStream_t st) {
    if constexpr (D == 64) {
        if (p.rows) return launch_rows<D, DT, CAUSAL, WLSE>(a, st);
    }
    if constexpr (FA2_MFMA_QG2 != 0 && D == 64) {
        if (p.qg == 2) return launch_q<D, DT, CAUSAL, WLSE, 2>(a, p, st);
    }
    return launch_q<D, DT, CAUSAL, WLSE, 1>(a, p, st);
}

template <int D, int DT>
fa2_status launch_dt(const FwdArgs &a, hipStream_t st) {
    const Plan p = plan(a.B, a.H, a.Nq, a.Nk, D, a.causal, a.num_cus);
    if (p.n_tiles < 0) return FA2_ERR_UNSUPPORTED;
    if (a.causal)
        return a.lse ? launch_v<D, DT, true, true>(a, p, st) : launch_v<D, DT, true, false>(a, p, st);
    return a.lse ? launch_v<D, DT, false, true>(a, p, st) : launch_v<D, DT, false, false>(a, p, st);
}

}  // namespace

fa2_status launch_fwd_mfma(const FwdArgs &a, fa2_dtype dt, hipStream_t st) {
    if (a.D == 128) return dt == FA2_F16 ? launch_dt<128, 1>(a, st) : launch_dt<128, 2>(a, st);
    return dt == FA2_F16 ? launch_dt<64, 1>(a, st) : launch_dt<64, 2>(a, st);
}

size_t mfma_workspace_bytes(int B, int H, int Nq, int Nk, int D, int causal, int num_cus) {
    const Plan p = plan(B, H, Nq, Nk, D, causal, num_cus);
    if (p.rows || p.chunks <= 1) return 0;
    if (p.chunks == 2) return PairLayout(p.n_tiles, kWaves * 32 * p.qg, D).bytes;
    return (size_t)B * H * Nq * p.chunks * (D + 3) * sizeof(float);
}

}  // namespace fa2
