// fwd_mfma.hip -- exact attention forward, f16 / bf16 in and out, D = 64, on
// gfx950 matrix cores (v_mfma_f32_32x32x16_{f16,bf16}), f32 softmax state.
//
// Method: the FlashAttention-2 forward ("Flash Attention" (aarnphm.xyz),
// sections Deriving the online softmax and FlashAttention 2; "06: Fused
// attention", attn_fwd).  A workgroup owns 128 query rows, one 32-row slab per
// wave (each wave owns whole rows, so no cross-wave reduction is needed), and
// walks the keys in blocks of 64 staged through LDS.  Per block and wave:
//     S^T = K Q^T                    (8 MFMAs, f32 accumulate)
//     m_new = max(m, rowmax S);  P = exp(S - m);  l = l*corr + rowsum P
//     O^T = corr*O^T + V^T P^T       (8 MFMAs, P rounded to the input dtype)
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
//   * O^T likewise holds 32 of the 64 output columns of that query, so corr and
//     1/l are per-lane scalars.
//   * The P registers feed the B operand of O^T = V^T P^T without moving:
//     16-key chunk c of key tile T uses registers 8c..8c+7 of tile T.  The
//     matching V^T operand comes from the row-major V block by the transposed
//     LDS read (ds_read_b64_tr_b16): lane i of each 16-lane group receives 4
//     keys of d = i when the group points at 4 keys x 4 groups of 4 columns.
//   * LDS rows (128 bytes) have their 16-byte chunks XOR-swizzled by key.
#include "fa2_device.h"
#include "fa2_internal.h"

namespace fa2 {

namespace {

constexpr int kD = 64;
constexpr int kBR = 128;     // query rows per workgroup
constexpr int kBC = 64;      // keys per block
constexpr int kWaves = 4;    // 32 query rows per wave
constexpr float kTau = 8.f;  // rescale threshold, base-2 units

// Tuning knobs (compile-time).  FA2_KSWZ selects the K-tile chunk swizzle:
// 1 = chunk ^ ((key/2) % 8), conflict-free for 16 lanes x 16 bytes over 64
// banks; 0 = chunk ^ (key % 8).  FA2_SCHED = 1 interleaves the next block's
// score MFMAs with the current block's softmax explicitly.
#ifndef FA2_KSWZ
#define FA2_KSWZ 1
#endif
#ifndef FA2_SCHED
#define FA2_SCHED 0
#endif

__device__ __forceinline__ int kswz(int key) { return FA2_KSWZ ? (key >> 1) & 7 : key & 7; }

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

template <int DT, bool CAUSAL>
__global__ __launch_bounds__(kWaves * 64, 3) void fwd_mfma_d64_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, uint16_t *__restrict__ O, float *__restrict__ LSE,
    int Nq, int Nk, float scale_log2, int n_qtiles, int n_tiles) {
    // Two K and two V buffers, as separate arrays (not one indexed array) so
    // the compiler can see that reads of one never alias DMA into another.
    __shared__ __attribute__((aligned(16))) uint16_t sK0[kBC * kD];
    __shared__ __attribute__((aligned(16))) uint16_t sK1[kBC * kD];
    __shared__ __attribute__((aligned(16))) uint16_t sV0[kBC * kD];
    __shared__ __attribute__((aligned(16))) uint16_t sV1[kBC * kD];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;
    const int ql = lane & 31;

    // Workgroups go round-robin to the 8 XCDs; give each XCD a contiguous run
    // of tiles so the query tiles of one head share that XCD's L2.
    int wg = blockIdx.x;
    if ((n_tiles & 7) == 0) wg = (wg & 7) * (n_tiles >> 3) + (wg >> 3);
    const int bh = wg / n_qtiles;
    int qt = wg - bh * n_qtiles;
    if (CAUSAL) qt = n_qtiles - 1 - qt;  // longest rows first
    const int q0 = qt * kBR;
    const int qw = q0 + wave * 32;  // first row of this wave
    const int myq = qw + ql;        // the query this lane's columns belong to

    const uint16_t *Qh = Q + (size_t)bh * Nq * kD;
    const uint16_t *Kh = K + (size_t)bh * Nk * kD;
    const uint16_t *Vh = V + (size_t)bh * Nk * kD;
    const auto rq = make_rsrc(Qh, (uint32_t)Nq * kD * 2);
    const auto rk = make_rsrc(Kh, (uint32_t)Nk * kD * 2);
    const auto rv = make_rsrc(Vh, (uint32_t)Nk * kD * 2);

    // B operand of S^T = K Q^T: chunk dc, slot (h, j) is Q[myq][16dc + 8h + j].
    u32x4 qf[4];
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) qf[dc] = load16(rq, (uint32_t)((myq * kD + 16 * dc + 8 * h) * 2));

    const int kend = CAUSAL ? min(Nk, q0 + kBR) : Nk;
    const int nblk = (kend + kBC - 1) / kBC;

    // Rows past Nk are never loaded with data; make sure the V rows they
    // would occupy hold zeros (0 * V must stay 0 for the masked keys).
    if (Nk % kBC != 0) {
        u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            reinterpret_cast<u32x4 *>(sV0)[tid + 256 * i] = z;
            reinterpret_cast<u32x4 *>(sV1)[tid + 256 * i] = z;
        }
        __syncthreads();
    }

    // HBM/L2 -> LDS: wave w moves 16-byte units [(2w+i)*64, +64) of the
    // block; unit P holds chunk (P%8) ^ swizzle(key) of key P/8 (swizzle kswz
    // for K, key % 8 for V).
    auto dma = [&](const __amdgpu_buffer_rsrc_t &r, uint16_t *dst, int k0, bool r_is_k) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int unit = (2 * wave + i) * 64 + lane;
            const int key = unit >> 3;
            const int ch = (unit & 7) ^ (r_is_k ? kswz(key) : (key & 7));
            const uint32_t off = (uint32_t)(((k0 + key) * kD + ch * 8) * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst + (2 * wave + i) * 512), 16,
                                                     off, 0, 0, 0);
        }
    };

    // LDS offsets that do not change from block to block.  Every key a lane
    // reads sits at a multiple of 8 from its first one, so the chunk swizzle
    // (key % 8) is fixed per lane and the rest is an immediate offset.
    int kofs[4], vofs[2];
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) kofs[dc] = ql * kD + (((2 * dc + h) ^ kswz(ql)) << 3);
    {
        const int i = lane & 15;
        const int kl = 4 * h + (i >> 2);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
            const int d = 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (i & 3);
            vofs[dt] = kl * kD + (((d >> 3) ^ kl) << 3) + (d & 7);
        }
    }

    auto scores = [&](const uint16_t *kb, f32x16 *s) {
#pragma unroll
        for (int T = 0; T < 2; ++T) {
#pragma unroll
            for (int i = 0; i < 16; ++i) s[T][i] = 0.f;
#pragma unroll
            for (int dc = 0; dc < 4; ++dc) {
                const u32x4 a = *reinterpret_cast<const u32x4 *>(&kb[kofs[dc] + 32 * T * kD]);
                s[T] = MfmaT<DT>::mma(a, qf[dc], s[T]);
            }
        }
    };

    float m = -INFINITY;  // max used for the exponentials, base-2 units
    float l = 0.f;        // this lane's half of the running denominator (f32 P)
    float lt = 0.f;       // the same over P as rounded for the MFMA
    const uint32_t ones = DT == 1 ? 0x3C003C00u : 0x3F803F80u;  // (1, 1) in f16 / bf16
    f32x16 oacc[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        oacc[0][i] = 0.f;
        oacc[1][i] = 0.f;
    }

    // Block j's K lives in sK[j % 2] and its V in sV[j % 2].  While block b is
    // computed, K_{b+2} and V_{b+1} stream in; they are waited for at the end
    // of block b.
    // Prologue: K_0, V_0, K_1 in and visible; scores of block 0.
    dma(rk, sK0, 0, true);
    dma(rv, sV0, 0, false);
    if (nblk > 1) dma(rk, sK1, kBC, true);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x16 sa[2], sb[2];
    scores(sK0, sa);

    // One block: on entry LDS holds K_{b+1} in kn and V_b in vc.  K_{b+2}
    // goes to kd (K_b's buffer) and V_{b+1} to vd (V_{b-1}'s), both last read
    // in the previous block.  scur holds the scores of block b; those of
    // block b+1 go to snext.
    auto step = [&](int b, const uint16_t *kn, uint16_t *kd, const uint16_t *vc, uint16_t *vd,
                    f32x16 *scur, f32x16 *snext) {
        const int k0 = b * kBC;
        if (b + 1 < nblk) dma(rv, vd, k0 + kBC, false);
        if (b + 2 < nblk) dma(rk, kd, k0 + 2 * kBC, true);

        // Without a causal mask every block is live for every wave, and the
        // scores of the next block are computed unconditionally (past the last
        // block they read a stale buffer and are never used) so that they share
        // one basic block with this block's softmax and P V and can interleave.
        const bool next_live = CAUSAL ? (b + 1 < nblk && k0 + kBC <= qw + 31) : true;
        const bool live = !(CAUSAL && k0 > qw + 31);
        if (live) {
            // scur[T][r] = S[myq][k0 + 32T + 8(r/4) + 4h + r%4]
            const bool need_mask = (k0 + kBC > Nk) || (CAUSAL && k0 + kBC - 1 > qw);
            if (need_mask) {
#pragma unroll
                for (int T = 0; T < 2; ++T)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + 32 * T + 8 * (r >> 2) + 4 * h + (r & 3);
                        bool ok = key < Nk;
                        if (CAUSAL) ok = ok && key <= myq;
                        if (!ok) scur[T][r] = -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int T = 0; T < 2; ++T)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, scur[T][r]);
            mx = max_halves(mx) * scale_log2;
            if (__builtin_amdgcn_ballot_w64(mx > m + kTau) != 0) {
                const float m_new = fmaxf(m, mx);
                const float corr = exp2f_fast(m - (m_new == -INFINITY ? 0.f : m_new));
                l *= corr;
                lt *= corr;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    oacc[0][i] *= corr;
                    oacc[1][i] *= corr;
                }
                m = m_new;
            }
            if (next_live) scores(kn, snext);
            const float m_use = m == -INFINITY ? 0.f : m;
            float psum = 0.f;
#pragma unroll
            for (int T = 0; T < 2; ++T)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    u32x4 pk;
#pragma unroll
                    for (int r = 8 * c; r < 8 * c + 8; r += 2) {
                        const float p0 = exp2f_fast(__builtin_fmaf(scur[T][r], scale_log2, -m_use));
                        const float p1 = exp2f_fast(__builtin_fmaf(scur[T][r + 1], scale_log2, -m_use));
                        const uint32_t w = pack2<DT>(p0, p1);
                        pk[(r & 7) >> 1] = w;
                        psum += p0 + p1;
                        lt = dot2<DT>(w, ones, lt);
                    }
#pragma unroll
                    for (int dt = 0; dt < 2; ++dt) {
                        const uint16_t *src = vc + vofs[dt] + (32 * T + 16 * c) * kD;
                        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)src);
                        const s16x4 hi =
                            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(src + 8 * kD));
                        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
                        const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
                        const u32x4 a = {lo2[0], lo2[1], hi2[0], hi2[1]};
                        oacc[dt] = MfmaT<DT>::mma(a, pk, oacc[dt]);
                    }
                }
            l += psum;
#if FA2_SCHED
            // 8 K reads, then score MFMAs each followed by VALU work, then the
            // V reads and the P V MFMAs likewise interleaved with VALU.
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
            }
#endif
        }
        // This block's DMA has landed; after the barrier every wave's has.
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
    };

    // Unrolled by 2 so every buffer and register choice is fixed at compile time.
    for (int b = 0; b < nblk; b += 2) {
        step(b, sK1, sK0, sV0, sV1, sa, sb);
        if (b + 1 < nblk) step(b + 1, sK0, sK1, sV1, sV0, sb, sa);
    }

    // oacc[dt][r] = O[myq][32dt + 8(r/4) + 4h + r%4] * l
    l += __shfl_xor(l, 32);
    lt += __shfl_xor(lt, 32);
    if (myq < Nq) {
        const float inv = 1.f / lt;
        uint16_t *orow = O + ((size_t)bh * Nq + myq) * kD;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = 32 * dt + 8 * g4 + 4 * h;
                const int r = 4 * g4;
                u32x2 w;
                w[0] = pack2<DT>(oacc[dt][r] * inv, oacc[dt][r + 1] * inv);
                w[1] = pack2<DT>(oacc[dt][r + 2] * inv, oacc[dt][r + 3] * inv);
                *reinterpret_cast<u32x2 *>(orow + d) = w;
            }
        if (LSE && h == 0) LSE[(size_t)bh * Nq + myq] = (m + log2f_fast(l)) * kLn2;
    }
}

template <int DT>
fa2_status launch_dt(const FwdArgs &a, hipStream_t st) {
    const int n_qtiles = (a.Nq + kBR - 1) / kBR;
    const long long n_tiles = (long long)n_qtiles * a.B * a.H;
    if (n_tiles > 0x7FFFFFFF) return FA2_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)n_tiles);
    const dim3 block(kWaves * 64);
    const float sl2 = a.scale * kLog2e;
    if (a.causal)
        return launch(fwd_mfma_d64_kernel<DT, true>, grid, block, st, (const uint16_t *)a.q,
                      (const uint16_t *)a.k, (const uint16_t *)a.v, (uint16_t *)a.o, a.lse, a.Nq,
                      a.Nk, sl2, n_qtiles, (int)n_tiles);
    return launch(fwd_mfma_d64_kernel<DT, false>, grid, block, st, (const uint16_t *)a.q,
                  (const uint16_t *)a.k, (const uint16_t *)a.v, (uint16_t *)a.o, a.lse, a.Nq,
                  a.Nk, sl2, n_qtiles, (int)n_tiles);
}

}  // namespace

fa2_status launch_fwd_mfma_d64(const FwdArgs &a, fa2_dtype dt, hipStream_t st) {
    return dt == FA2_F16 ? launch_dt<1>(a, st) : launch_dt<2>(a, st);
}

}  // namespace fa2
