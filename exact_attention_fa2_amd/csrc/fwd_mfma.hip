// fwd_mfma.hip -- exact attention forward, f16 / bf16 in and out, D = 64, on
// gfx950 matrix cores (v_mfma_f32_32x32x16_{f16,bf16}), f32 softmax state.
//
// Method: the FlashAttention-2 forward ("Flash Attention" (aarnphm.xyz),
// sections Deriving the online softmax and FlashAttention 2; "06: Fused
// attention", attn_fwd).  A workgroup owns 128 query rows, one 32-row slab per
// wave (each wave owns whole rows, so no cross-wave reduction is needed), and
// walks the keys in blocks of 64 staged through LDS.  Per block and wave:
//     S^T = K Q^T                    (8 MFMAs, f32 accumulate)
//     m_new = max(m, rowmax S);  P = exp(S - m_new);  corr = exp(m - m_new)
//     l = l*corr + rowsum P;      O^T = corr*O^T + V^T P^T   (8 MFMAs)
// with P rounded to the input dtype for the second product.  After the last
// block O = O/l is rounded to the output dtype and LSE = m + ln l is stored.
// Causal: blocks wholly above a wave's diagonal are skipped and only blocks
// that cross it are masked ("Flash Attention", note on causal masking).
//
// Register layouts (32x32 MFMA accumulator: lane l, register r holds row
// 8*(r/4) + 4*(l/32) + r%4, column l%32):
//   * S^T has keys as rows and queries as columns, so lane l holds 32 scores of
//     ONE query (l%32); its partner lane l^32 holds the other 32.  Row max needs
//     a single cross-lane step and the running denominator none until the end.
//   * O^T likewise holds 32 of the 64 output columns of that same query, so the
//     rescale by corr and the final 1/l are per-lane scalars.
//   * The P accumulator registers feed the B operand of O^T = V^T P^T without
//     moving: chunk c of 16 keys uses registers 8c..8c+7.  The matching V^T
//     operand is read from an LDS copy of V stored transposed, with key index
//     bits 2 and 3 swapped so each lane's 8 keys are 16 contiguous bytes.
//   * LDS rows are XOR-swizzled in 16-byte units against bank conflicts.
#include "fa2_device.h"
#include "fa2_internal.h"

namespace fa2 {

namespace {

constexpr int kD = 64;
constexpr int kBR = 128;   // query rows per workgroup
constexpr int kBC = 64;    // keys per block
constexpr int kWaves = 4;  // 32 query rows per wave

template <int DT>
struct MfmaT;
template <>
struct MfmaT<1> {
    typedef half8 v8;
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

// LDS element offsets (16-bit units).  K: [key][d], 16-byte chunk swizzled by key.
__device__ __forceinline__ int k_off(int key, int chunk) {
    return key * kD + ((chunk ^ (key & 7)) << 3);
}
// V^T: [d][position], position = key with bits 2,3 swapped, chunk swizzled by d.
__device__ __forceinline__ int vt_chunk_off(int d, int chunk) {
    return d * kBC + ((chunk ^ (d & 7) ^ ((d >> 3) & 7)) << 3);
}

template <int DT, bool CAUSAL>
__global__ __launch_bounds__(kWaves * 64, 2) void fwd_mfma_d64_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, uint16_t *__restrict__ O, float *__restrict__ LSE,
    int Nq, int Nk, float scale_log2, int n_qtiles, int n_tiles) {
    __shared__ __attribute__((aligned(16))) uint16_t sK[kBC * kD];
    __shared__ __attribute__((aligned(16))) uint16_t sV[kD * kBC];

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

    // Staging: thread t moves K/V rows t/8 and 32 + t/8, 16-byte chunk t%8.
    const int srow = tid >> 3, sch = tid & 7;
    u32x4 kreg[2], vreg[2];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const uint32_t off = (uint32_t)(((k0 + srow + 32 * it) * kD + sch * 8) * 2);
            kreg[it] = load16(rk, off);
            vreg[it] = load16(rv, off);
        }
    };
    fetch(0);

    float m = -INFINITY;  // running max, base-2 units of the scaled score
    float l = 0.f;        // this lane's half of the running denominator
    f32x16 oacc[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        oacc[0][i] = 0.f;
        oacc[1][i] = 0.f;
    }

    for (int b = 0; b < nblk; ++b) {
        const int k0 = b * kBC;
        __syncthreads();  // every wave is done with the previous block
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int key = srow + 32 * it;
            *reinterpret_cast<u32x4 *>(&sK[k_off(key, sch)]) = kreg[it];
            const int pos = (int)swap_bits23((uint32_t)key);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int d = sch * 8 + i;
                const uint32_t w = vreg[it][i >> 1];
                sV[vt_chunk_off(d, pos >> 3) + (pos & 7)] = (uint16_t)((i & 1) ? (w >> 16) : (w & 0xFFFF));
            }
        }
        __syncthreads();
        if (b + 1 < nblk) fetch(k0 + kBC);

        if (CAUSAL && k0 > qw + 31) continue;  // every key of this block is masked for this wave

        f32x16 sacc[2];
#pragma unroll
        for (int T = 0; T < 2; ++T) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[T][i] = 0.f;
#pragma unroll
            for (int dc = 0; dc < 4; ++dc) {
                const u32x4 a = *reinterpret_cast<const u32x4 *>(&sK[k_off(32 * T + ql, 2 * dc + h)]);
                sacc[T] = MfmaT<DT>::mma(a, qf[dc], sacc[T]);
            }
        }
        // sacc[T][r] = S[myq][k0 + 32T + 8(r/4) + 4h + r%4]
        const bool need_mask = (k0 + kBC > Nk) || (CAUSAL && k0 + kBC - 1 > qw);
        if (need_mask) {
#pragma unroll
            for (int T = 0; T < 2; ++T)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 32 * T + 8 * (r >> 2) + 4 * h + (r & 3);
                    bool live = key < Nk;
                    if (CAUSAL) live = live && key <= myq;
                    if (!live) sacc[T][r] = -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[T][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m, mx * scale_log2);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float corr = exp2f_fast(m - m_use);
        float psum = 0.f;
        u32x4 pk[2][2];
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = exp2f_fast(__builtin_fmaf(sacc[T][r], scale_log2, -m_use));
                const float p1 = exp2f_fast(__builtin_fmaf(sacc[T][r + 1], scale_log2, -m_use));
                psum += p0 + p1;
                pk[T][r >> 3][(r & 7) >> 1] = pack2<DT>(p0, p1);
            }
        l = l * corr + psum;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            oacc[0][i] *= corr;
            oacc[1][i] *= corr;
        }
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int chunk = 2 * (2 * T + c) + h;
#pragma unroll
                for (int dt = 0; dt < 2; ++dt) {
                    const int d = 32 * dt + ql;
                    const u32x4 a = *reinterpret_cast<const u32x4 *>(&sV[vt_chunk_off(d, chunk)]);
                    oacc[dt] = MfmaT<DT>::mma(a, pk[T][c], oacc[dt]);
                }
            }
        m = m_new;
    }

    // oacc[dt][r] = O[myq][32dt + 8(r/4) + 4h + r%4] * l
    l += __shfl_xor(l, 32);
    if (myq < Nq) {
        const float inv = 1.f / l;
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
