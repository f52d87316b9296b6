// fwd_f32.hip -- exact attention forward, float32 in and out, D = 64 or 128,
// on the float32 matrix cores of gfx950 (v_mfma_f32_16x16x4_f32: full f32
// operands, f32 accumulation; nothing is rounded to a narrower type).
//
// Method ("Flash attention, f32": sections One block of queries per CTA, The
// loop over keys, Online softmax, After the loop; "Flash Attention"
// (aarnphm.xyz): Deriving the online softmax, tile form).  A workgroup owns
// one or two blocks of 16 query rows, read from memory once into LDS and from
// there into every wave's registers.  Its waves (16 with one block at D = 64,
// else 8) each walk a contiguous slice of the workgroup's keys, 16 keys a
// step, carrying a running max m, the running denominator l and the
// unnormalised output O.  O and l are rescaled by exp(m_old - m_new) only when
// a step's scores overtake m far enough that some exp(s - m) would pass 2^8
// (or the row has no m yet); below that, keeping the older m changes only the
// common factor of O and l, which the final O/l cancels.  At the end the
// waves' partial states are merged with the (m, l) monoid of "Flash
// Attention" (section Deriving the online softmax) through LDS, then O/l and
// LSE = m + ln l are written -- or, when a tile's keys were split between two
// workgroups, the two states are merged the same way by the second of them
// to finish.
//
// Why split the keys across waves: one head of 4096 rows gives only 256 tiles
// of 16 rows, or 128 of 32; splitting each tile's keys among the workgroup's
// waves puts two to four waves on every SIMD, enough to keep the matrix cores
// fed while other waves wait for their K/V loads, and with 32-row tiles the
// keys are also split between two workgroups so that every compute unit has
// one.  The pages' FlashAttention-2 prefers splitting queries across warps
// ("Flash Attention", section FlashAttention 2); these kernels keep that
// across workgroups where there are enough rows.
//
// A third kernel, for many query rows, shares each K/V block between four
// 16-row tiles through LDS (namespace shared below).
//
// Lane layout (lane = 16*g + c):
//   S^T = K Q^T per 16-key step: lane holds scores of query c for keys 4g..4g+3;
//   MFMA i pairs K and Q at d = 16*(i/4) + 4g + i%4 in lane group g.
//   O^T = V^T P^T: lane holds O[query c][16g .. 16g+15] (the MFMA's n index is
//   permuted so that each lane's V operand is one 16-byte row segment).
// The contraction index of both products is only a pairing of operand slots,
// so A and B just have to agree on it.
#include <algorithm>

#include "fa2_device.h"
#include "fa2_internal.h"

namespace fa2 {

namespace {

constexpr int kD = 64;
constexpr int kQT = 16;     // query rows of a row block (one 16x16 MFMA tile)
constexpr int kWaves = 16;  // waves of a shared-K/V workgroup (4 per SIMD)
constexpr int kStep = 16;   // keys per step
// A step's exponentials are kept, taken against the running max as it stands,
// when each lane's four P values sum to at most this (every P <= 2^8, far from
// f32 overflow); otherwise the step's max is taken, O and l are rescaled and
// the exponentials taken again.
constexpr float kLazyCap = 256.f;

// Query tile and head of this workgroup.  The grid is one-dimensional with
// b*h varying fastest: consecutive workgroups take the same query tile of
// different heads, so under a causal mask they have the same length, and the
// longest tiles go first.  Workgroups reach the XCDs (and, within one, its
// shader engines) in turn; with the query tile varying fastest instead, each
// shader engine would get the same few tiles of every head and the one holding
// the last tiles would carry a full unmasked load.  With b*h a multiple of 8,
// each XCD also sees only every eighth head, and its L2 holds their K and V.
template <bool CAUSAL>
__device__ __forceinline__ void tile_of(int n_qtiles, int index, int count, int &qt, int &bh) {
    const int n_bh = count / n_qtiles;
    qt = index / n_bh;
    bh = index - qt * n_bh;
    if (CAUSAL) qt = n_qtiles - 1 - qt;
}

// Grid of n_qtiles query tiles for each of n_bh heads (chunks key chunks).
inline dim3 tile_grid(long long n_qtiles, long long n_bh, int chunks) {
    return dim3((unsigned)(n_qtiles * n_bh), 1, (unsigned)chunks);
}

// Row-tile kernel shapes.  RB blocks of 16 query rows per workgroup, W waves
// each walking a contiguous slice of the workgroup's keys:
//   D = 64,  RB = 1: 16 waves (four per SIMD, 128 registers each);
//   D = 64,  RB = 2: 8 waves (two per SIMD, 164 registers): every K/V operand
//                    a wave loads feeds both row blocks, so loads per flop and
//                    the per-step vector work halve;
//   D = 128, RB = 1: 8 waves (the K/V operands double, 256 registers).
template <int D, int RB>
constexpr int rows_waves() {
    return D == 64 && RB == 1 ? 16 : 8;
}

template <int D>
struct KVRegs {
    f32x4 k[D / 16];     // k[j] = K[key k0 + c][16j + 4g .. 16j + 4g + 3]
    f32x4 v[4][D / 64];  // v[t][h] = V[key k0 + 4g + t][64h + 4c .. 64h + 4c + 3], t = 0..3
};

// The 16 keys from k0 on.  The buffer descriptors start at key k0 and cover
// the keys left (none past Nk), so the per-lane offsets stay the same from
// step to step and the step's position is scalar arithmetic on the
// descriptor; keys at or past Nk read as zeros.
template <int D>
__device__ __forceinline__ void load_kv(KVRegs<D> &r, const float *Kh, const float *Vh, int Nk,
                                        int k0, int g, int c) {
    const int kb = k0 < Nk ? k0 : Nk;  // base within the tensor; no records past Nk
    const uint32_t bytes = (uint32_t)(Nk - kb) * D * 4;
    const auto rk = make_rsrc(Kh + (size_t)kb * D, bytes);
    const auto rv = make_rsrc(Vh + (size_t)kb * D, bytes);
#pragma unroll
    for (int j = 0; j < D / 16; ++j)
        r.k[j] = __builtin_bit_cast(f32x4, load16(rk, (uint32_t)((c * D + 16 * j + 4 * g) * 4)));
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int h = 0; h < D / 64; ++h)
            r.v[t][h] = __builtin_bit_cast(
                f32x4, load16(rv, (uint32_t)(((4 * g + t) * D + 64 * h + 4 * c) * 4)));
}

// The workgroup's state after its waves are merged, per row: O unnormalised
// (kD floats), then m (base 2) and l -- one workgroup's share of the keys,
// written for the workgroup that merges the key chunks of a tile.
template <int QT, int D>
constexpr int part_floats() {
    return QT * D + 2 * QT;
}

// Row-tile kernel.  A workgroup owns RB * 16 query rows and one of NCH
// contiguous chunks of their keys; its W waves split that chunk.  With
// NCH = 2 ("Flash decoding": split the keys, keep unnormalised partials,
// merge them with the (m, l) monoid of "Flash Attention"), the two
// workgroups of a tile meet at the end without waiting for each other: each
// writes its partial state to `part`, then swaps `tag` (a 64-bit value drawn
// for this launch) into the tile's handshake word; the one that gets `tag`
// back is second, merges both states and writes O and LSE, and sets the word
// to 0 again.  The partial state goes through system-scope stores and loads
// (written through to memory and read from it, past every cache), and the
// swap is a system-scope atomic issued only after those stores have
// completed, so neither side needs a cache-wide write-back or invalidate
// (a fence would do both to the whole L2 of the XCD).
template <int D, bool CAUSAL, int RB, int NCH>
__global__ __launch_bounds__((rows_waves<D, RB>() * 64), 1) void fwd_f32_rows_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    float *__restrict__ O, float *__restrict__ LSE, int Nq, int Nk, float scale_log2,
    float *__restrict__ part, unsigned long long *__restrict__ tags, unsigned long long tag) {
    constexpr int W = rows_waves<D, RB>();
    constexpr int NH = D / 64;  // 64-column halves of O
    constexpr int QT = kQT * RB;  // query rows of the workgroup
    // score accumulation chains per row block: with one block, two
    // independent chains (summed at the end) keep the matrix core busy
    constexpr int NCHAIN = RB == 1 ? 2 : 1;
    static_assert(NCH == 1 || (D == 64 && QT * D / 4 == W * 64), "the chunk merge maps one f32x4 per thread");
    __shared__ __attribute__((aligned(16))) float s_o[W][QT][D];
    __shared__ float s_m[W][QT];
    __shared__ float s_l[W][QT];
    __shared__ float s_mg[QT], s_lg[QT];  // the workgroup's merged m and l (chunked launches)
    __shared__ int s_second;

    const int lane = threadIdx.x & 63;
    // wave index as a wave-uniform value, so the key loop below is scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, c = lane & 15;
    const int n_qtiles = (Nq + QT - 1) / QT;
    const int unit = blockIdx.x / NCH, chunk = blockIdx.x - unit * NCH;
    int qt, bh;
    tile_of<CAUSAL>(n_qtiles, unit, gridDim.x / NCH, qt, bh);
    const int q0 = qt * QT;

    const float *Qh = Q + (size_t)bh * Nq * D;
    const float *Kh = K + (size_t)bh * Nk * D;
    const float *Vh = V + (size_t)bh * Nk * D;
    const auto rq = make_rsrc(Qh, (uint32_t)Nq * D * 4);

    // Q^T operand of S^T = K Q^T: slot i of lane (g,c) in row block b is
    // Q[q0 + 16b + c][d(g,i)] with d(g,i) = 16*(i/4) + 4g + i%4 -- any pairing
    // of the contraction index works, and this one lets the four lanes of a
    // key row read 64 contiguous bytes of K per load instruction.
    // The row maxima below are taken on unscaled scores, which needs a
    // positive scale: a negative one moves onto Q (an exact sign flip) and a
    // zero one becomes Q = 0 with scale 1 (the scaled scores are the same).
    const float qmul = scale_log2 < 0.f ? -1.f : scale_log2 == 0.f ? 0.f : 1.f;
    scale_log2 = scale_log2 == 0.f ? 1.f : fabsf(scale_log2);

    // This workgroup's keys: chunk `chunk` of the tile's steps; then this
    // wave's contiguous share of them (possibly none).
    const int kend = CAUSAL ? min(Nk, q0 + QT) : Nk;
    const int nsteps = (kend + kStep - 1) / kStep;
    const int csteps = (nsteps + NCH - 1) / NCH;
    const int cs0 = min(nsteps, chunk * csteps);
    const int cs1 = min(nsteps, cs0 + csteps);
    const int per = (cs1 - cs0 + W - 1) / W;
    const int st0 = cs0 + wave * per;
    const int st1 = min(cs1, st0 + per);

    // This wave's first K/V operands go out before Q, the larger load first.
    KVRegs<D> ra, rb;
    load_kv<D>(ra, Kh, Vh, Nk, st0 * kStep, g, c);

    // The workgroup's Q tile is read from memory once, through the merge area
    // of LDS (free until the end), instead of once per wave.
    {
        float *sq = &s_o[0][0][0];
        for (int e = threadIdx.x; e < QT * D / 4; e += W * 64)
            *reinterpret_cast<f32x4 *>(sq + 4 * e) = __builtin_bit_cast(f32x4, load16(rq, (uint32_t)((q0 * D + 4 * e) * 4)));
        __syncthreads();
    }
    float qv[RB][D / 4];
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int j = 0; j < D / 16; ++j) {
            const f32x4 t = *reinterpret_cast<const f32x4 *>(&s_o[0][0][0] + (16 * b + c) * D + 16 * j + 4 * g);
            qv[b][4 * j + 0] = t[0] * qmul;
            qv[b][4 * j + 1] = t[1] * qmul;
            qv[b][4 * j + 2] = t[2] * qmul;
            qv[b][4 * j + 3] = t[3] * qmul;
        }
    // every wave has its Q before the merge area is written again
    __syncthreads();

    float m[RB], mu[RB], l[RB];  // per row block: running max of scaled scores
                                 // (base 2), that max or 0 while the row has no
                                 // live key yet, this lane's share of l
    f32x4 acc[RB][4 * NH];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
        m[b] = -INFINITY;
        mu[b] = 0.f;
        l[b] = 0.f;
#pragma unroll
        for (int j = 0; j < 4 * NH; ++j) acc[b][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // One 16-key step on the registers in `cur`; the next step's K/V are
    // loaded into `nxt` first so the loads overlap this step's work.  The load
    // is issued on every step, also the last (it then reads past this wave's
    // keys, harmlessly: in-slice data or zeros from the buffer descriptor), so
    // the compiler's count of loads in flight is the same on every path and its
    // wait for `cur` never also waits for `nxt`.
    auto step = [&](int st, const KVRegs<D> &cur, KVRegs<D> &nxt) {
        const int k0 = st * kStep;
        load_kv<D>(nxt, Kh, Vh, Nk, k0 + kStep, g, c);
        // keep the loads here: without this the scheduler sinks them next to
        // their use in the following step, which serialises load and compute
        __builtin_amdgcn_sched_barrier(0);

        f32x4 sacc[RB][NCHAIN];
#pragma unroll
        for (int b = 0; b < RB; ++b)
#pragma unroll
            for (int ch = 0; ch < NCHAIN; ++ch) sacc[b][ch] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < D / 4; i += NCHAIN)
#pragma unroll
            for (int b = 0; b < RB; ++b)
#pragma unroll
                for (int ch = 0; ch < NCHAIN; ++ch)
                    sacc[b][ch] = __builtin_amdgcn_mfma_f32_16x16x4f32(cur.k[(i + ch) >> 2][(i + ch) & 3],
                                                                      qv[b][i + ch], sacc[b][ch], 0, 0, 0);
        if constexpr (NCHAIN == 2) {
#pragma unroll
            for (int b = 0; b < RB; ++b) sacc[b][0] += sacc[b][1];
        }

        // sacc[b][0][r] = S[query q0 + 16b + c][key k0 + 4g + r] (unscaled); a
        // step past this wave's slice is masked entirely and leaves the state
        // unchanged.  Only steps that reach past Nk, cross the causal diagonal
        // or lie past the slice need the per-score mask (a wave-uniform test).
        float s[RB][4];
        const bool in_slice = st < st1;
        if (in_slice && k0 + kStep <= Nk && !(CAUSAL && k0 + kStep - 1 > q0)) {
#pragma unroll
            for (int b = 0; b < RB; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) s[b][r] = sacc[b][0][r];
        } else {
#pragma unroll
            for (int b = 0; b < RB; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = k0 + 4 * g + r;
                    bool live = in_slice && key < Nk;
                    if (CAUSAL) live = live && key <= q0 + 16 * b + c;
                    s[b][r] = live ? sacc[b][0][r] : -INFINITY;
                }
        }
        float p[RB][4], psum[RB];
        bool need = false;
#pragma unroll
        for (int b = 0; b < RB; ++b) {
#pragma unroll
            for (int r = 0; r < 4; ++r) p[b][r] = exp2f_fast(__builtin_fmaf(s[b][r], scale_log2, -mu[b]));
            psum[b] = (p[b][0] + p[b][1]) + (p[b][2] + p[b][3]);
            need = need || m[b] == -INFINITY || psum[b] > kLazyCap;
        }
        // The max is only taken (and O rescaled) when a row has none yet or a
        // score has overtaken it far enough to push some P past the cap; a
        // rescale by exactly 1 would change nothing.
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
            for (int b = 0; b < RB; ++b) {
                float mx = fmax_nan(fmax_nan(s[b][0], s[b][1]), fmax_nan(s[b][2], s[b][3]));
                mx = max_xor32(max_xor16(mx)) * scale_log2;  // base-2 units of the scaled scores
                const float m_new = fmax_nan(m[b], mx);
                mu[b] = m_new == -INFINITY ? 0.f : m_new;
                const float corr = exp2f_fast(m[b] - mu[b]);
                l[b] *= corr;
#pragma unroll
                for (int j = 0; j < 4 * NH; ++j) acc[b][j] *= corr;
                m[b] = m_new;
#pragma unroll
                for (int r = 0; r < 4; ++r) p[b][r] = exp2f_fast(__builtin_fmaf(s[b][r], scale_log2, -mu[b]));
                psum[b] = (p[b][0] + p[b][1]) + (p[b][2] + p[b][3]);
            }
        }
#pragma unroll
        for (int b = 0; b < RB; ++b) l[b] += psum[b];
        // O^T += V^T P^T: slot g pairs key k0 + 4g + t; row m of tile 4h + j is
        // d = 64h + 4m + j.
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int b = 0; b < RB; ++b)
#pragma unroll
                for (int h = 0; h < NH; ++h)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[b][4 * h + j] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                            cur.v[t][h][j], p[b][t], acc[b][4 * h + j], 0, 0, 0);
    };

    // Steps run in pairs, unconditionally, so each step's prefetch has a
    // use on every path and the compiler keeps it where it is issued.
    for (int st = st0; st < st1; st += 2) {
        step(st, ra, rb);
        step(st + 1, rb, ra);
    }

    // acc[b][4h + j][r] = O[q0 + 16b + c][64h + 16g + 4r + j]; the lane's l
    // covers keys 4g..4g+3 of each step.
#pragma unroll
    for (int b = 0; b < RB; ++b) {
        float lb = l[b];
        lb += __shfl_xor(lb, 16);
        lb += __shfl_xor(lb, 32);
        if (g == 0) {
            s_m[wave][16 * b + c] = m[b];
            s_l[wave][16 * b + c] = lb;
        }
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                *reinterpret_cast<f32x4 *>(&s_o[wave][16 * b + c][64 * h + 16 * g + 4 * r]) =
                    f32x4{acc[b][4 * h][r], acc[b][4 * h + 1][r], acc[b][4 * h + 2][r], acc[b][4 * h + 3][r]};
    }
    __syncthreads();

    // Merge the wave states of each row ((m, l) merge of the online softmax).
    // First W lanes per row, one per wave state: the row's max m by a
    // reduction over those lanes, each state's weight 2^(m_w - m), and l as
    // the weighted sum of the states' l.  The weights replace the row's s_m
    // entries; the row's m and l go to s_mg, s_lg, and s_l[0][row] holds 1 / l
    // (each row's lanes sit in one wave and read their entries before any of
    // them is written).
    if (threadIdx.x < QT * W) {
        const int row = threadIdx.x / W, w = threadIdx.x % W;
        const float mw = s_m[w][row];
        const float mg = group_reduce<W, true>(mw);
        const float wt = mw == -INFINITY ? 0.f : exp2f_fast(mw - mg);
        const float lg = group_reduce<W>(wt * s_l[w][row]);
        s_m[w][row] = wt;
        if (w == 0) {
            s_mg[row] = mg;
            s_lg[row] = lg;
            s_l[0][row] = 1.f / lg;
            const int qrow = q0 + row;
            if (NCH == 1 && LSE && qrow < Nq) LSE[(size_t)bh * Nq + qrow] = (mg + log2f_fast(lg)) * kLn2;
        }
    }
    __syncthreads();
    if constexpr (NCH == 1) {
        // Four consecutive output columns per thread: the weighted sum of the
        // states' O, divided by l once.
        for (int e = threadIdx.x; e < QT * D / 4; e += W * 64) {
            const int row = e / (D / 4);
            const int d = 4 * (e % (D / 4));
            f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < W; ++w) o += s_m[w][row] * *reinterpret_cast<const f32x4 *>(&s_o[w][row][d]);
            const int qrow = q0 + row;
            if (qrow < Nq) *reinterpret_cast<f32x4 *>(O + ((size_t)bh * Nq + qrow) * D + d) = o * s_l[0][row];
        }
    } else {
        // One f32x4 of the workgroup's unnormalised O per thread.
        const int row = threadIdx.x / (D / 4);
        const int d = 4 * (threadIdx.x % (D / 4));
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < W; ++w) o += s_m[w][row] * *reinterpret_cast<const f32x4 *>(&s_o[w][row][d]);

        // Publish this chunk's state (cache policy 17 = SC0 | SC1, system
        // scope), wait until every store of the workgroup has completed, then
        // swap the tag.
        constexpr int kSys = 17;
        constexpr int PF = part_floats<QT, D>();
        const auto rmine = make_rsrc(part + ((size_t)unit * NCH + chunk) * PF, PF * 4);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rmine, (row * D + d) * 4, 0, kSys);
        if (d == 0) {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s_mg[row]), rmine, (QT * D + row) * 4, 0, kSys);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s_lg[row]), rmine, (QT * D + QT + row) * 4, 0, kSys);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0) {
            const unsigned long long old =
                __hip_atomic_exchange(&tags[unit], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            const int second = old == tag;
            if (second)  // ready for the next launch
                __hip_atomic_exchange(&tags[unit], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            s_second = second;
        }
        __syncthreads();
        if (!s_second) return;

        // Second: merge the two chunks' states in chunk order (the same
        // arithmetic whichever workgroup does it) and write O and LSE.
        const auto rother = make_rsrc(part + ((size_t)unit * NCH + (chunk ^ 1)) * PF, PF * 4);
        const f32x4 oo = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rother, (row * D + d) * 4, 0, kSys));
        const float mo = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rother, (QT * D + row) * 4, 0, kSys));
        const float lo = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rother, (QT * D + QT + row) * 4, 0, kSys));
        const float mm = s_mg[row], lm = s_lg[row];
        const bool c0 = chunk == 0;
        const float m0 = c0 ? mm : mo, m1 = c0 ? mo : mm;
        const float l0 = c0 ? lm : lo, l1 = c0 ? lo : lm;
        const f32x4 o0 = c0 ? o : oo, o1 = c0 ? oo : o;
        const float mg = fmax_nan(m0, m1);
        const float w0 = m0 == -INFINITY ? 0.f : exp2f_fast(m0 - mg);
        const float w1 = m1 == -INFINITY ? 0.f : exp2f_fast(m1 - mg);
        const float lg = w0 * l0 + w1 * l1;
        const int qrow = q0 + row;
        if (qrow < Nq) {
            *reinterpret_cast<f32x4 *>(O + ((size_t)bh * Nq + qrow) * D + d) = (w0 * o0 + w1 * o1) * (1.f / lg);
            if (LSE && d == 0) LSE[(size_t)bh * Nq + qrow] = (mg + log2f_fast(lg)) * kLn2;
        }
    }
}

// ---------------------------------------------------------------------------
// Shared-K/V variant with an optional split of the keys across workgroups.
//
// A workgroup owns 64 query rows (4 tiles of 16) and one chunk of the keys.
// Its 16 waves are 4 query tiles x 4 key sub-slices; each K/V block of a
// sub-slice is moved into LDS once (DMA) and read by the 4 waves of the 4
// query tiles, so every byte fetched from L2 feeds 64 rows instead of 16.
// When the keys are split into C chunks ("Flash decoding": split the keys,
// keep unnormalised partials, merge with the (m, l) monoid), each workgroup
// writes (O_s, m_s, l_s) for its rows and chunk and the decode combine kernel
// merges them; with C = 1 it writes O and LSE itself.
namespace shared {

constexpr int kTiles = 4;                   // query tiles of 16 rows per workgroup
constexpr int kSub = kWaves / kTiles;       // key sub-slices per workgroup
constexpr int kRows = kTiles * kQT;         // 64 query rows per workgroup
constexpr int kBlkBytes = kStep * kD * 4;   // 4 KB: one 16-key block of K (or V)
constexpr int kBufBytes = kSub * 2 * kBlkBytes;  // K and V blocks of all sub-slices

typedef __attribute__((address_space(3))) void lds_void;

template <bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(kWaves * 64, 1) void kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    float *__restrict__ O, float *__restrict__ LSE, float *__restrict__ o_part,
    float *__restrict__ m_part, float *__restrict__ l_part, int Nq, int Nk, float scale_log2) {
    // Two K/V buffers (separate arrays, so DMA into one is seen not to alias
    // reads of the other); after the loop the same 64 KB hold the merge.
    __shared__ __attribute__((aligned(16))) char buf0[kBufBytes];
    __shared__ __attribute__((aligned(16))) char buf1[kBufBytes];
    __shared__ float s_m[kWaves][kQT];
    __shared__ float s_l[kWaves][kQT];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int qa = wave & (kTiles - 1);  // query tile of this wave
    const int ss = wave / kTiles;        // key sub-slice of this wave
    const int g = lane >> 4, c = lane & 15;
    int qt, bh;
    tile_of<CAUSAL>((Nq + kRows - 1) / kRows, blockIdx.x, gridDim.x, qt, bh);
    const int q0 = qt * kRows;
    const int chunk = blockIdx.z, nchunks = gridDim.z;
    const int qt0 = q0 + qa * kQT;  // first row of this wave's tile

    const float *Qh = Q + (size_t)bh * Nq * kD;
    const float *Kh = K + (size_t)bh * Nk * kD;
    const float *Vh = V + (size_t)bh * Nk * kD;
    const auto rq = make_rsrc(Qh, (uint32_t)Nq * kD * 4);
    const auto rk = make_rsrc(Kh, (uint32_t)Nk * kD * 4);
    const auto rv = make_rsrc(Vh, (uint32_t)Nk * kD * 4);

    // Q^T operand, pairing d = 16*(i/4) + 4g + i%4 as in the kernel above,
    // with the sign of the scale moved onto Q as there.
    const float qmul = scale_log2 < 0.f ? -1.f : scale_log2 == 0.f ? 0.f : 1.f;
    scale_log2 = scale_log2 == 0.f ? 1.f : fabsf(scale_log2);
    float qv[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f32x4 t = __builtin_bit_cast(f32x4, load16(rq, (uint32_t)(((qt0 + c) * kD + 16 * j + 4 * g) * 4)));
        qv[4 * j + 0] = t[0] * qmul;
        qv[4 * j + 1] = t[1] * qmul;
        qv[4 * j + 2] = t[2] * qmul;
        qv[4 * j + 3] = t[3] * qmul;
    }

    // Steps of 16 keys: the chunk's steps, then this sub-slice's share.
    const int kend = CAUSAL ? min(Nk, q0 + kRows) : Nk;
    const int nsteps = (kend + kStep - 1) / kStep;
    const int per_chunk = (nsteps + nchunks - 1) / nchunks;
    const int c0 = chunk * per_chunk;
    const int c1 = min(nsteps, c0 + per_chunk);
    const int per_sub = max(0, (c1 - c0 + kSub - 1) / kSub);
    auto sub_first = [&](int sub) { return c0 + sub * per_sub; };
    const int st0 = sub_first(ss);
    const int st1 = min(c1, st0 + per_sub);

    // DMA of iteration `it` into a buffer: instruction I = 2*wave + i covers
    // 1 KB; sub-slice I/8, part I%8 (0-3: K rows 4p..4p+3, 4-7: V rows).  K
    // rows keep their 16-byte chunks XOR-swizzled by row, V rows are linear.
    auto dma = [&](char *dst, int it) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int I = 2 * wave + i;
            const int sub = I >> 3, part = I & 7;
            const bool is_k = part < 4;
            const int unit = (part & 3) * 64 + lane;  // 16-byte unit in the 4 KB block
            const int row = unit >> 4, phys = unit & 15;
            const int logical = is_k ? (phys ^ row) : phys;
            const int key = (sub_first(sub) + it) * kStep + row;
            // keys past the slice get an offset past the descriptor's range
            // (zeros; never used): computed so that nothing can overflow
            const uint32_t off =
                key < Nk ? (uint32_t)key * (kD * 4) + (uint32_t)logical * 16 : 0xFFFFFFF0u;
            char *blk = dst + (sub * 2 + (is_k ? 0 : 1)) * kBlkBytes;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(is_k ? rk : rv, (lds_void *)(blk + (part & 3) * 1024),
                                                     16, off, 0, 0, 0);
        }
    };

    float m = -INFINITY, mu = 0.f, l = 0.f;  // mu: m, or 0 while m is -inf
    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // This step's K and V operands, read from LDS into registers.
    auto fetch = [&](const char *bufc, f32x4 *kr, f32x4 *vr) {
        const char *kb = bufc + (ss * 2) * kBlkBytes;
        const char *vb = kb + kBlkBytes;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            kr[j] = *reinterpret_cast<const f32x4 *>(kb + c * 256 + (((4 * j + g) ^ c) << 4));
#pragma unroll
        for (int t = 0; t < 4; ++t)
            vr[t] = *reinterpret_cast<const f32x4 *>(vb + (4 * g + t) * 256 + (c << 4));
    };

    auto step = [&](const f32x4 *kr, const f32x4 *vr, int it) {
        const int st = st0 + it;
        const int k0 = st * kStep;

        f32x4 sacc = {0.f, 0.f, 0.f, 0.f}, sacc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[i >> 2][i & 3], qv[i], sacc, 0, 0, 0);
            sacc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[i >> 2][(i & 3) + 1], qv[i + 1], sacc2,
                                                        0, 0, 0);
        }
        sacc += sacc2;
        // unscaled scores, masked only on steps that need it; then the
        // exponentials against the running max, kept unless the max must move
        // (the rule of the kernel above)
        const bool in_slice = st < st1;
        float sv[4];
        if (in_slice && k0 + kStep <= Nk && !(CAUSAL && k0 + kStep - 1 > qt0)) {
#pragma unroll
            for (int r = 0; r < 4; ++r) sv[r] = sacc[r];
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = k0 + 4 * g + r;
                bool live = in_slice && key < Nk;
                if (CAUSAL) live = live && key <= qt0 + c;
                sv[r] = live ? sacc[r] : -INFINITY;
            }
        }
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = exp2f_fast(__builtin_fmaf(sv[r], scale_log2, -mu));
        float psum = (p[0] + p[1]) + (p[2] + p[3]);
        if (__builtin_amdgcn_ballot_w64(m == -INFINITY || psum > kLazyCap) != 0) {
            float mx = fmax_nan(fmax_nan(sv[0], sv[1]), fmax_nan(sv[2], sv[3]));
            mx = max_xor32(max_xor16(mx)) * scale_log2;
            const float m_new = fmax_nan(m, mx);
            mu = m_new == -INFINITY ? 0.f : m_new;
            const float corr = exp2f_fast(m - mu);
            l *= corr;
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] *= corr;
            m = m_new;
#pragma unroll
            for (int r = 0; r < 4; ++r) p[r] = exp2f_fast(__builtin_fmaf(sv[r], scale_log2, -mu));
            psum = (p[0] + p[1]) + (p[2] + p[3]);
        }
        l += psum;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(vr[t][j], p[t], acc[j], 0, 0, 0);
    };

    // Iterations: every sub-slice advances one step per iteration.  On entry
    // to iteration it the buffer for it is in LDS; the DMA for it+1 goes to
    // the other buffer, last read in iteration it-1.
    // The operands are read before the next DMA is issued: a read that comes
    // after an LDS DMA in program order would make the compiler wait for that
    // DMA, which it cannot tell writes the other buffer.
    dma(buf0, 0);
    f32x4 kr[4], vr[4];
    for (int it = 0; it < per_sub; it += 2) {
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
        fetch(buf0, kr, vr);
        if (it + 1 < per_sub) dma(buf1, it + 1);
        step(kr, vr, it);
        if (it + 1 < per_sub) {
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_s_barrier();
            fetch(buf1, kr, vr);
            if (it + 2 < per_sub) dma(buf0, it + 2);
            step(kr, vr, it + 1);
        }
    }

    // Merge the 4 sub-slice states of each row through LDS.
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // every wave is done with the K/V buffers
    // [16 rows][64] floats per wave: waves 0-7 in buf0, 8-15 in buf1
    static_assert(sizeof(buf0) >= (kWaves / 2) * kQT * kD * 4, "merge space");
    auto wave_o = [&](int w) {
        return reinterpret_cast<float *>(w < kWaves / 2 ? buf0 : buf1) + (w % (kWaves / 2)) * kQT * kD;
    };
    if (g == 0) {
        s_m[wave][c] = m;
        s_l[wave][c] = l;
    }
    {
        float *mine = wave_o(wave);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            *reinterpret_cast<f32x4 *>(&mine[c * kD + 16 * g + 4 * r]) =
                f32x4{acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
    }
    __syncthreads();

    // 1024 threads, 64 rows x 64 columns: 4 consecutive columns per thread.
    const int row = threadIdx.x >> 4;         // 0..63
    const int d = (threadIdx.x & 15) * 4;
    const int tile = row / kQT, rr = row % kQT;
    float mg = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub) mg = fmaxf(mg, s_m[sub * kTiles + tile][rr]);
    float lg = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub) {
        const int w = sub * kTiles + tile;
        const float mw = s_m[w][rr];
        const float wt = mw == -INFINITY ? 0.f : exp2f_fast(mw - mg);
        lg += wt * s_l[w][rr];
        o += wt * *reinterpret_cast<const f32x4 *>(&wave_o(w)[rr * kD + d]);
    }
    const int qrow = q0 + row;
    if (qrow >= Nq) return;
    const size_t rowid = (size_t)bh * Nq + qrow;
    if (!SPLIT) {
        *reinterpret_cast<f32x4 *>(O + rowid * kD + d) = o / lg;
        if (LSE && d == 0) LSE[rowid] = (mg + log2f_fast(lg)) * kLn2;
    } else {
        const size_t pidx = rowid * nchunks + chunk;
        *reinterpret_cast<f32x4 *>(o_part + pidx * kD + d) = o;
        if (d == 0) {
            m_part[pidx] = mg == -INFINITY ? -INFINITY : mg * kLn2;  // natural-log units
            l_part[pidx] = lg;
        }
    }
}

}  // namespace shared

}  // namespace

// Split plan for the shared kernel: number of key chunks (1 = no split).
// Split only when even 16-row workgroups cannot cover the device: with one
// 16-row workgroup per compute unit or more, the unsplit kernels measured
// faster than split + combine.
#ifndef FA2_F32_SPLIT_BELOW
#define FA2_F32_SPLIT_BELOW 1  // split while 16-row tiles < this many per compute unit
#endif
#ifndef FA2_F32_SPLIT_WAVES
#define FA2_F32_SPLIT_WAVES 1  // chunks so that groups x chunks = this many per compute unit
#endif
// 1: D = 64 shapes with at least one 64-row group per compute unit run the
// shared-K/V kernel; 0: they run the row-tile kernels.
#ifndef FA2_F32_SHARED
#define FA2_F32_SHARED 1
#endif
// 1: unmasked D = 64 shapes with too few 64-row groups for the shared kernel
// run the 32-row kernel (its keys split in two and merged in the kernel when
// the 32-row tiles cover only half the device); 0: the 16-row kernel.
#ifndef FA2_F32_ROWS32
#define FA2_F32_ROWS32 1
#endif

int f32_chunks(int B, int H, int Nq, int Nk, int num_cus) {
    const long long groups = (long long)B * H * ((Nq + shared::kRows - 1) / shared::kRows);
    const long long tiles16 = (long long)B * H * ((Nq + kQT - 1) / kQT);
    if (groups >= num_cus || tiles16 >= (long long)FA2_F32_SPLIT_BELOW * num_cus) return 1;
    const int nsteps = (Nk + kStep - 1) / kStep;
    long long c = ((long long)FA2_F32_SPLIT_WAVES * num_cus + groups - 1) / groups;
    c = std::min<long long>(c, std::max(1, nsteps / shared::kSub));  // >= one step per sub-slice
    c = std::min<long long>(c, 64);
    return (int)std::max<long long>(1, c);
}

namespace {

constexpr int kRows32 = 2 * kQT;  // query rows of the 32-row kernel's workgroup

// Which D = 64 kernel a shape gets.
enum class F32Plan { Shared, Rows32, Rows32Split, SharedSplit, Rows16 };

// Unmasked shapes whose 32-row tiles, split in two, cover the device take
// whichever row-tile schedule should finish first.  Workgroups run in rounds
// of one per compute unit, so a schedule costs its rounds times the time of
// one workgroup, counted per SIMD in steps of 16 keys for 16 rows:
//   16-row tiles:       4 waves x ceil(n / 16) steps
//   32-row tiles:       2 waves x ceil(n / 8) steps x 2 blocks x 0.9
//   32-row, keys split: 2 waves x ceil(ceil(n / 2) / 8) steps x 2 x 0.9 + 3
// (n = steps of the keys; a 32-row step takes 0.9 of two 16-row steps,
// measured on one head of 4096 x 4096: 36.5 against 40.3 us per launch
// before the merge; the merge of a split tile costs about 3 steps, 1.8 us).
// The split is taken only when it should save at least 3% (below that the
// model cannot tell, and the split needs a workspace of 16.5 KB per tile).
// This picked the faster schedule on every shape measured, and the 32-row
// kernel also beat the shared-K/V kernel on every many-row shape (by 3-21%).
// Causal shapes keep the 16-row and shared-K/V kernels: their tiles differ
// in length, and with 32-row tiles the longest ones set the time (single
// head of 8192, causal: 127 against 88 us).  So do shapes with fewer rows,
// which split the keys across 64-row groups and merge with the combine.
F32Plan f32_plan(int B, int H, int Nq, int Nk, int causal, int num_cus, bool have_ws) {
    const long long bh = (long long)B * H;
    const long long groups = bh * ((Nq + shared::kRows - 1) / shared::kRows);
    const long long t16 = bh * ((Nq + kQT - 1) / kQT);
    const long long t32 = bh * ((Nq + kRows32 - 1) / kRows32);
    if (FA2_F32_ROWS32 && !causal && 2 * t32 >= num_cus) {
        auto rounds = [&](long long wgs) { return (double)((wgs + num_cus - 1) / num_cus); };
        const long long n = (Nk + kStep - 1) / kStep;
        const double c16 = rounds(t16) * 4.0 * ((n + 15) / 16);
        const double c32 = rounds(t32) * 3.6 * ((n + 7) / 8);
        const double c32s = rounds(2 * t32) * (3.6 * (((n + 1) / 2 + 7) / 8) + 3.0);
        if (have_ws && c32s < 0.97 * std::min(c16, c32)) return F32Plan::Rows32Split;
        return c32 < c16 ? F32Plan::Rows32 : F32Plan::Rows16;
    }
    if (FA2_F32_SHARED && groups >= num_cus) return F32Plan::Shared;
    return f32_chunks(B, H, Nq, Nk, num_cus) > 1 ? F32Plan::SharedSplit : F32Plan::Rows16;
}

// Workspace of the 32-row kernel with its keys split in two: a 64-bit
// handshake word per tile (the words padded to 256 bytes), then two partial
// states per tile.
struct Rows32SplitLayout {
    size_t words, bytes;
    explicit Rows32SplitLayout(long long tiles)
        : words(((size_t)tiles * 8 + 255) / 256 * 256),
          bytes(words + (size_t)tiles * 2 * part_floats<kRows32, kD>() * sizeof(float)) {}
};

}  // namespace

size_t f32_workspace_bytes(int B, int H, int Nq, int Nk, int D, int causal, int num_cus) {
    if (D != kD) return 0;  // D = 128 always runs the 16-row kernel
    switch (f32_plan(B, H, Nq, Nk, causal, num_cus, true)) {
        case F32Plan::Rows32Split:
            return Rows32SplitLayout((long long)B * H * ((Nq + kRows32 - 1) / kRows32)).bytes;
        case F32Plan::SharedSplit: {
            const int c = f32_chunks(B, H, Nq, Nk, num_cus);
            return (size_t)B * H * Nq * c * (kD + 2) * sizeof(float);
        }
        default:
            return 0;
    }
}

// The row-tile kernel on a one-dimensional grid of NCH workgroups per tile
// (chunk fastest), b*h next, query tile slowest.
template <int D, int RB, int NCH>
fa2_status launch_rows(const FwdArgs &a, float sl2, hipStream_t st, float *part = nullptr,
                       unsigned long long *tags = nullptr, unsigned long long tag = 0) {
    constexpr int QT = kQT * RB;
    const long long units = (long long)((a.Nq + QT - 1) / QT) * a.B * a.H;
    const dim3 grid((unsigned)(units * NCH));
    const dim3 block(rows_waves<D, RB>() * 64);
    if constexpr (RB == 1) {
        auto k = a.causal ? fwd_f32_rows_kernel<D, true, 1, NCH> : fwd_f32_rows_kernel<D, false, 1, NCH>;
        return launch(k, grid, block, st, (const float *)a.q, (const float *)a.k, (const float *)a.v,
                      (float *)a.o, a.lse, a.Nq, a.Nk, sl2, part, tags, tag);
    } else {
        if (a.causal) return FA2_ERR_UNSUPPORTED;  // the planner sends only unmasked shapes here
        return launch(fwd_f32_rows_kernel<D, false, RB, NCH>, grid, block, st, (const float *)a.q,
                      (const float *)a.k, (const float *)a.v,
                      (float *)a.o, a.lse, a.Nq, a.Nk, sl2, part, tags, tag);
    }
}

fa2_status launch_fwd_f32(const FwdArgs &a, hipStream_t st) {
    // one-dimensional grids of 16-row tiles (the most numerous) must fit a grid dimension
    if ((long long)a.B * a.H * ((a.Nq + kQT - 1) / kQT) > 0x7FFFFFFFLL) return FA2_ERR_UNSUPPORTED;
    const float sl2 = a.scale * kLog2e;
    // D = 128: the 16-row kernel at two waves per SIMD for every shape (the
    // shared-K/V kernel holds the operands of four query tiles per wave group
    // and has no registers for twice the columns)
    if (a.D == 128) return launch_rows<128, 1, 1>(a, sl2, st);
    const dim3 block(kWaves * 64);
    const size_t need = f32_workspace_bytes(a.B, a.H, a.Nq, a.Nk, kD, a.causal, a.num_cus);
    const bool ws_ok = need > 0 && a.ws && a.ws_bytes >= need;
    const F32Plan plan = f32_plan(a.B, a.H, a.Nq, a.Nk, a.causal, a.num_cus, ws_ok);
    if (plan == F32Plan::Shared) {
        // enough 64-row groups to fill the device: share K/V, no split
        const dim3 grid = tile_grid((a.Nq + shared::kRows - 1) / shared::kRows, a.B * a.H, 1);
        auto k = a.causal ? shared::kernel<true, false> : shared::kernel<false, false>;
        return launch(k, grid, block, st, (const float *)a.q, (const float *)a.k, (const float *)a.v,
                      (float *)a.o, a.lse, (float *)nullptr, (float *)nullptr, (float *)nullptr,
                      a.Nq, a.Nk, sl2);
    }
    if (plan == F32Plan::Rows32) return launch_rows<kD, 2, 1>(a, sl2, st);
    if (plan == F32Plan::Rows32Split) {
        // each 32-row tile's keys in two chunks, merged by the second of its
        // two workgroups
        const Rows32SplitLayout lay((long long)a.B * a.H * ((a.Nq + kRows32 - 1) / kRows32));
        auto *tags = (unsigned long long *)a.ws;
        float *part = (float *)((char *)a.ws + lay.words);
        return launch_rows<kD, 2, 2>(a, sl2, st, part, tags, next_launch_tag());
    }
    if (plan == F32Plan::SharedSplit && ws_ok) {
        // few rows: split the keys into c chunks, then merge the partials
        const int c = f32_chunks(a.B, a.H, a.Nq, a.Nk, a.num_cus);
        const size_t rows = (size_t)a.B * a.H * a.Nq;
        float *o_part = (float *)a.ws;
        float *m_part = o_part + rows * c * kD;
        float *l_part = m_part + rows * c;
        const dim3 grid = tile_grid((a.Nq + shared::kRows - 1) / shared::kRows, a.B * a.H, c);
        auto k = a.causal ? shared::kernel<true, true> : shared::kernel<false, true>;
        fa2_status s = launch(k, grid, block, st, (const float *)a.q, (const float *)a.k,
                              (const float *)a.v, (float *)a.o, a.lse, o_part, m_part, l_part, a.Nq,
                              a.Nk, sl2);
        if (s != FA2_OK) return s;
        return launch_combine_rows(o_part, m_part, l_part, a.o, a.lse, rows, kD, c, FA2_F32, st);
    }
    // few rows and no workspace: 16-row workgroups fill the device instead
    return launch_rows<kD, 1, 1>(a, sl2, st);
}

}  // namespace fa2
