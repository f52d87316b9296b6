// bwd.hip -- exact attention backward, f16 / bf16, D = 64 or 128, on gfx950
// matrix cores, float32 accumulation.
//
// Method ("Flash Attention" (aarnphm.xyz), section IO complexity, the
// paragraph on the backward pass; "06: Fused attention", the backward
// kernels): only O and the per-row log-sum-exp L are kept from the forward;
// the probabilities are recomputed block by block as P = exp(scale S - L),
// and with D_i = rowsum(dO o O)
//     dV = P^T dO,   dP = dO V^T,   dS = P o (dP - D_i),
//     dQ = scale dS K,   dK = scale dS^T Q.
// Three kernels: D (one pass over O and dO), dQ (a workgroup per 128 query
// rows walking the keys), dK/dV (a workgroup per 128 keys -- 64 with D = 128,
// where two waves share 32 keys and split the output columns -- walking the
// queries).  P and dS are rounded to the input dtype before their MFMAs, as
// P is in the forward.
//
// Layouts are those of the forward kernel (32x32x16 MFMA, accumulator lane l
// register r = row 8(r/4) + 4(l/32) + r%4, column l%32):
//   dQ kernel:  S^T = K Q^T and D - dP^T = V (-dO)^T + D (keys x queries,
//               one query per lane), dQ^T -= K^T (-dS^T) with K^T read by the
//               transposed LDS load;
//   dK/dV:      S = Q K^T and D - dP = dO (-V)^T + D (queries x keys, one key
//               per lane), dV^T += dO^T P and dK^T -= Q^T (-dS), dO^T and Q^T
//               transposed from LDS.
// (dO, resp. V, is negated once in registers so that the product starts
// from D and no per-element subtraction is needed; the sign of dS is undone
// in the final scale.)
// Every LDS tile is read both by rows (b128) and transposed (tr_b16); its
// 16-byte chunks are swizzled so that neither read has bank conflicts.
#include <type_traits>

#include "fa2_device.h"
#include "fa2_internal.h"

// Waves per SIMD the dK/dV kernel is compiled for (its register budget),
// without and with causal masking.
#ifndef FA2_BWD_KV_OCC
#define FA2_BWD_KV_OCC 3
#endif
#ifndef FA2_BWD_KV_OCC_CAUSAL
#define FA2_BWD_KV_OCC_CAUSAL 2
#endif
// Order of the two 32-row halves of a staged block: 1 issues the second
// half's products before the first half's exponentials (more overlap, more
// registers), 0 runs the halves one after the other.  Per kernel: dQ, dK/dV.
#ifndef FA2_BWD_PIPE_Q
#define FA2_BWD_PIPE_Q 1
#endif
#ifndef FA2_BWD_PIPE_KV
#define FA2_BWD_PIPE_KV 0
#endif

namespace fa2 {

namespace {

constexpr int kWaves = 4;
constexpr int kRows = 128;  // query rows a dQ workgroup owns (32 per wave); keys of a D = 64 dK/dV one
constexpr int kBlk = 64;    // rows of the other side staged per block

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

template <int DT>
__device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (DT == 1)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                                      __builtin_bit_cast(half8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 16-byte chunk swizzle of the LDS tiles: logical chunk c of row r sits in
// slot c ^ swz(r).  Tiles here are read both by rows (b128, 16 lanes per
// pass) and transposed (tr_b16, 32 lanes per pass over 4 consecutive rows).
// D = 64 (128-byte rows, two per 64 banks): rows of one parity within 16 need
// distinct swz, rows r and r + 2 swz differing in bit 2; j ^ 4(j & 1) with
// j = (r / 2) % 8 meets both.  D = 128 (a row spans the 64 banks): swz must
// permute 16 chunks over any 16 rows and send 4 consecutive rows to different
// aligned groups of four; 4(r % 4) + (r / 4) % 4 does.
template <int D>
__device__ __forceinline__ int swz(int row) {
    if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
    const int j = (row >> 1) & 7;
    return j ^ ((j & 1) << 2);
}

// Tile offsets (16-bit elements) of a swizzled D-column row-major LDS tile.
//   row_ofs[dc]:  A operand "rows x d" of MFMA chunk dc: lane reads row ql,
//                 chunk 2dc + h.
//   tr_ofs[dt][u]: A operand "d x rows" (transposed read) of the 32 columns
//                 from dbase + 32 dt: lane group i of 16 gets 4 rows of
//                 column d, in rows kl (u = 0) and kl + 8 (u = 1); add 16c
//                 rows for contraction chunk c.
template <int D, int NTR>
struct TileOfs {
    int row_ofs[D / 16], tr_ofs[NTR][2];
    __device__ __forceinline__ TileOfs(int lane, int dbase) {
        const int h = lane >> 5, ql = lane & 31;
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) row_ofs[dc] = ql * D + (((2 * dc + h) ^ swz<D>(ql)) << 3);
        const int i = lane & 15;
        const int kl = 4 * h + (i >> 2);
#pragma unroll
        for (int dt = 0; dt < NTR; ++dt) {
            const int d = dbase + 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (i & 3);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int row = kl + 8 * u;
                tr_ofs[dt][u] = row * D + (((d >> 3) ^ swz<D>(row)) << 3) + (d & 7);
            }
        }
    }
};

__device__ __forceinline__ u32x4 read_row(const uint16_t *tile, int ofs) {
    return *reinterpret_cast<const u32x4 *>(tile + ofs);
}

// Transposed A operand for contraction chunk c (16 rows) and d tile dt.
template <int D>
__device__ __forceinline__ u32x4 read_tr(const uint16_t *tile, const int *ofs, int c) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(tile + ofs[0] + 16 * c * D));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(tile + ofs[1] + 16 * c * D));
    const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
    const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
}

// HBM/L2 -> LDS of the 64 rows starting at row r0 of a [rows][D] tensor:
// wave w moves 16-byte units [(U w + i) 64, +64), U = D / 32; unit P holds
// chunk (P % (D/8)) ^ swz(row) of row P / (D/8).  Rows past the descriptor's
// range load nothing.
template <int D>
__device__ __forceinline__ void dma_tile(const __amdgpu_buffer_rsrc_t &r, uint16_t *dst, int r0,
                                         int wave, int lane) {
    constexpr int U = D / 32, CPR = D / 8;
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const int unit = (U * wave + i) * 64 + lane;
        const int row = unit / CPR;
        const int ch = (unit % CPR) ^ swz<D>(row);
        const uint32_t off = (uint32_t)(((r0 + row) * D + ch * 8) * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst + (U * wave + i) * 512), 16, off,
                                                 0, 0, 0);
    }
}

// ---------------------------------------------------------------------------
// D_i = sum_d dO_id O_id, float32; D/8 lanes per row, each 16 bytes.  Grid:
// (ceil(Nq / (256 / (D/8))), B*H).
template <int D, int DT>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const uint16_t *__restrict__ O,
                                                        const uint16_t *__restrict__ dO,
                                                        float *__restrict__ Delta, int Nq) {
    constexpr int LPR = D / 8;
    constexpr int kD = D;
    const int row = (blockIdx.x * 256 + threadIdx.x) / LPR;
    const int c = threadIdx.x % LPR;
    const size_t base = (size_t)blockIdx.y * Nq;
    float acc = 0.f;
    if (row < Nq) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(O + (base + row) * kD + 8 * c);
        const u32x4 b = *reinterpret_cast<const u32x4 *>(dO + (base + row) * kD + 8 * c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float a0, a1, b0, b1;
            unpack2<DT>(a[i], a0, a1);
            unpack2<DT>(b[i], b0, b1);
            acc = __builtin_fmaf(a0, b0, acc);
            acc = __builtin_fmaf(a1, b1, acc);
        }
    }
    acc = group_reduce<LPR>(acc);
    if (row < Nq && c == 0) Delta[base + row] = acc;
}

// ---------------------------------------------------------------------------
// dQ: a workgroup owns 128 query rows (32 per wave) of one (b,h) and walks
// the keys in 64-key blocks (K and V double-buffered in LDS).
template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(kWaves * 64, 2) void bwd_dq_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const uint16_t *__restrict__ dO, const float *__restrict__ LSE, const float *__restrict__ Delta,
    uint16_t *__restrict__ dQ, int BH, int Nq, int Nk, float scale, float scale_log2) {
    constexpr int kD = D, NC = D / 16, NT = D / 32;
    constexpr bool PIPE = FA2_BWD_PIPE_Q && D == 64;  // D = 128 has no registers for it
    // two buffers of 64 rows each for K and for V (block b in buffer b % 2)
    __shared__ __attribute__((aligned(16))) uint16_t sK[2 * kBlk * kD];
    __shared__ __attribute__((aligned(16))) uint16_t sV[2 * kBlk * kD];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, ql = lane & 31;
    // Workgroup w takes head w % BH and query block w / BH, counted from the
    // last block when causal (the longest first).  Workgroups of one head are
    // BH apart, a multiple of 8 when BH is, and so share one XCD's L2.
    const int nqb = (Nq + kRows - 1) / kRows;
    const int bh = blockIdx.x % BH;
    const int qb = blockIdx.x / BH;
    const int q0 = (CAUSAL ? nqb - 1 - qb : qb) * kRows;
    const int qw = q0 + 32 * wave;
    const int myq = qw + ql;

    const auto rq = make_rsrc(Q + (size_t)bh * Nq * kD, (uint32_t)Nq * kD * 2);
    const auto rdo = make_rsrc(dO + (size_t)bh * Nq * kD, (uint32_t)Nq * kD * 2);
    const auto rk = make_rsrc(K + (size_t)bh * Nk * kD, (uint32_t)Nk * kD * 2);
    const auto rv = make_rsrc(V + (size_t)bh * Nk * kD, (uint32_t)Nk * kD * 2);

    // B operands: chunk dc, slot (h, j) = Q[myq][16dc + 8h + j] and -dO[..]
    // (sign bits flipped, exact): the dP product then starts from D and
    // yields D - dP, with the sign carried into the final scale of dQ.
    u32x4 qf[NC], gf[NC];
#pragma unroll
    for (int dc = 0; dc < NC; ++dc) {
        qf[dc] = load16(rq, (uint32_t)((myq * kD + 16 * dc + 8 * h) * 2));
        gf[dc] = load16(rdo, (uint32_t)((myq * kD + 16 * dc + 8 * h) * 2)) ^ 0x80008000u;
    }
    const bool qlive = myq < Nq;
    const float l2 = qlive ? LSE[(size_t)bh * Nq + myq] * kLog2e : 0.f;  // base-2 units
    const float dlt = qlive ? Delta[(size_t)bh * Nq + myq] : 0.f;

    const int kend = CAUSAL ? min(Nk, q0 + kRows) : Nk;
    const int nblk = (kend + kBlk - 1) / kBlk;
    const TileOfs<D, NT> to(lane, 0);

    if (Nk % kBlk != 0) {  // rows past Nk are never loaded: keep them finite
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < D / 16; ++i) {
            reinterpret_cast<u32x4 *>(sK)[tid + 256 * i] = z;
            reinterpret_cast<u32x4 *>(sV)[tid + 256 * i] = z;
        }
        __syncthreads();
    }

    f32x16 acc[NT];  // dQ^T: acc[dt][r] = -dQ[myq][32dt + 8(r/4) + 4h + r%4] / scale
#pragma unroll
    for (int dt = 0; dt < NT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;

    // S^T and D - dP^T of one 32-key tile (rows kt / vt of the staged
    // block): s[r], dn[r] belong to key k0 + 8(r/4) + 4h + r%4 and query myq.
    auto prod = [&](const uint16_t *kt, const uint16_t *vt, f32x16 &s, f32x16 &dn) {
        f32x16 d0;
#pragma unroll
        for (int i = 0; i < 16; ++i) d0[i] = dlt;
#pragma unroll
        for (int dc = 0; dc < NC; ++dc) {
            s = mma<DT>(read_row(kt, to.row_ofs[dc]), qf[dc], dc == 0 ? f32x16{} : s);
            dn = mma<DT>(read_row(vt, to.row_ofs[dc]), gf[dc], dc == 0 ? d0 : dn);
        }
    };
    // -dS^T = P^T o (D - dP^T), rounded and packed as the B operand of dQ^T.
    // Keys past Nk and (causal) keys after the query get P = 0 when MASK.
    auto softgrad = [&](auto mask_tag, int k0, const f32x16 &s, const f32x16 &dn, u32x4 *pk)
        __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float ds2[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int r = 8 * c + 2 * j + e;
                    float x = __builtin_fmaf(s[r], scale_log2, -l2);
                    if constexpr (MASK) {
                        const int key = k0 + 8 * (r >> 2) + 4 * h + (r & 3);
                        bool live = key < Nk;
                        if (CAUSAL) live = live && key <= myq;
                        x = live ? x : -INFINITY;
                    }
                    ds2[e] = exp2f_fast(x) * dn[r];
                }
                pk[c][j] = pack2<DT>(ds2[0], ds2[1]);
            }
    };
    // dQ^T += K^T dS^T (K^T by the transposed read of the staged keys)
    auto grad = [&](const uint16_t *kt, const u32x4 *pk) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int dt = 0; dt < NT; ++dt) acc[dt] = mma<DT>(read_tr<D>(kt, to.tr_ofs[dt], c), pk[c], acc[dt]);
    };
    // One staged 64-key block: tiles A (keys kb..kb+31) and B (kb+32..).  B's
    // products are issued before A's exponentials and A's dQ products before
    // B's, so the matrix cores have work while the vector ALUs run.
    auto compute = [&](auto mask_tag, int kb, const uint16_t *kc, const uint16_t *vc, bool doB) {
        f32x16 sA, dA, sB, dB;
        u32x4 pA[2], pB[2];
        prod(kc, vc, sA, dA);
        if (PIPE && doB) prod(kc + 32 * kD, vc + 32 * kD, sB, dB);
        // D = 128: phase by phase, or the operand reads hoisted across the
        // phases run out of registers
        if constexpr (D == 128) __builtin_amdgcn_sched_barrier(0);
        softgrad(mask_tag, kb, sA, dA, pA);
        if constexpr (D == 128) __builtin_amdgcn_sched_barrier(0);
        grad(kc, pA);
        if (doB) {
            // keeps the scheduler from hoisting the second half's operand
            // reads above the first half (which runs out of registers)
            __builtin_amdgcn_sched_barrier(0);
            if (!PIPE) prod(kc + 32 * kD, vc + 32 * kD, sB, dB);
            if constexpr (D == 128) __builtin_amdgcn_sched_barrier(0);
            softgrad(mask_tag, kb + 32, sB, dB, pB);
            if constexpr (D == 128) __builtin_amdgcn_sched_barrier(0);
            grad(kc + 32 * kD, pB);
        }
    };

    if (nblk > 0) {
        dma_tile<D>(rk, sK, 0, wave, lane);
        dma_tile<D>(rv, sV, 0, wave, lane);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    // One staged block; MASK selects the masked path (keys past Nk, and
    // with causal masking keys after this wave's rows, including whole
    // tiles past its last row).
    auto block = [&](auto mask_tag, int b, const uint16_t *kc, const uint16_t *vc, uint16_t *kd,
                     uint16_t *vd) {
        constexpr bool MASK = decltype(mask_tag)::value;
        if (b + 1 < nblk) {
            dma_tile<D>(rk, kd, (b + 1) * kBlk, wave, lane);
            dma_tile<D>(rv, vd, (b + 1) * kBlk, wave, lane);
        }
        const int kb = b * kBlk;
        if constexpr (MASK) {
            // causal: tiles wholly after this wave's last query are skipped
            const bool doA = !CAUSAL || kb <= qw + 31;
            const bool doB = !CAUSAL || kb + 32 <= qw + 31;
            if (doA) compute(std::true_type{}, kb, kc, vc, doB);
        } else {
            compute(std::false_type{}, kb, kc, vc, true);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    // The blocks that need no mask come first (all keys < Nk and, causal,
    // <= this wave's first row): they run in a loop of their own, the rest
    // in a second one, so each loop has one copy of the block and its
    // accumulators stay in place (one loop with both paths made the compiler
    // copy them every block).  D = 128 masks every block: a second copy does
    // not fit its registers, and the mask's vector work hides under the
    // twice larger products.  Waves may split at different blocks; each
    // still passes one barrier per block.
    int bm = D == 128 ? 0 : min(nblk, Nk / kBlk);
    if (CAUSAL) bm = min(bm, (qw + 1) / kBlk);
    int b = 0;
    for (; b < bm; ++b) {
        const int cur = (b & 1) * kBlk * kD, nxt = kBlk * kD - cur;
        block(std::false_type{}, b, sK + cur, sV + cur, sK + nxt, sV + nxt);
    }
    for (; b < nblk; ++b) {
        const int cur = (b & 1) * kBlk * kD, nxt = kBlk * kD - cur;
        block(std::true_type{}, b, sK + cur, sV + cur, sK + nxt, sV + nxt);
    }

    if (qlive) {
        const float nscale = -scale;  // the accumulated dS had its sign flipped
        uint16_t *row = dQ + ((size_t)bh * Nq + myq) * kD;
#pragma unroll
        for (int dt = 0; dt < NT; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int r = 4 * g4;
                u32x2 w;
                w[0] = pack2<DT>(acc[dt][r] * nscale, acc[dt][r + 1] * nscale);
                w[1] = pack2<DT>(acc[dt][r + 2] * nscale, acc[dt][r + 3] * nscale);
                *reinterpret_cast<u32x2 *>(row + 32 * dt + 8 * g4 + 4 * h) = w;
            }
    }
}

// ---------------------------------------------------------------------------
// dK, dV: a workgroup owns 128 keys (32 per wave) of one (b,h) and walks the
// queries in 64-row tiles (Q, dO, L and D staged in LDS, double-buffered).
// With D = 128 a workgroup owns 64 keys: waves 2g and 2g + 1 take keys
// 32g .. 32g + 31, each forms S and D - dP over all 128 columns and keeps
// the dK, dV accumulators of its own 64 output columns (the full 128 would
// not fit two waves per SIMD).
template <int D>
constexpr int kv_keys_per_wg() { return D == 64 ? 128 : 64; }

template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(kWaves * 64, D == 128 ? 2 : (CAUSAL ? FA2_BWD_KV_OCC_CAUSAL : FA2_BWD_KV_OCC)) void bwd_dkdv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const uint16_t *__restrict__ dO, const float *__restrict__ LSE, const float *__restrict__ Delta,
    uint16_t *__restrict__ dK, uint16_t *__restrict__ dV, int BH, int Nq, int Nk, float scale,
    float scale_log2) {
    constexpr int kD = D, NC = D / 16;
    constexpr int KPW = kv_keys_per_wg<D>();
    // two buffers of 64 rows each for Q, dO and (L, D) (tile t in buffer t % 2)
    __shared__ __attribute__((aligned(16))) uint16_t sQ[2 * kBlk * kD];
    __shared__ __attribute__((aligned(16))) uint16_t sG[2 * kBlk * kD];
    __shared__ __attribute__((aligned(16))) float sL[2 * 2 * kBlk];  // L then D of 64 rows

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, ql = lane & 31;
    // Workgroup w takes head w % BH and key block w / BH (with causal masking
    // the first key blocks see the most queries, so they start first).
    const int bh = blockIdx.x % BH;
    const int k0 = (blockIdx.x / BH) * KPW;
    const int kg = D == 64 ? wave : wave >> 1;          // key group of this wave
    const int dbase = D == 64 ? 0 : 64 * (wave & 1);   // first output column it keeps
    const int kw = k0 + 32 * kg;  // first key of this wave
    const int myk = kw + ql;

    const auto rq = make_rsrc(Q + (size_t)bh * Nq * kD, (uint32_t)Nq * kD * 2);
    const auto rdo = make_rsrc(dO + (size_t)bh * Nq * kD, (uint32_t)Nq * kD * 2);
    const auto rk = make_rsrc(K + (size_t)bh * Nk * kD, (uint32_t)Nk * kD * 2);
    const auto rv = make_rsrc(V + (size_t)bh * Nk * kD, (uint32_t)Nk * kD * 2);
    const auto rl = make_rsrc(LSE + (size_t)bh * Nq, (uint32_t)Nq * 4);
    const auto rd = make_rsrc(Delta + (size_t)bh * Nq, (uint32_t)Nq * 4);

    // B operands: chunk dc, slot (h, j) = K[myk][16dc + 8h + j] and -V[..]
    // (sign bits flipped, exact): the dP product then starts from D and
    // yields D - dP, with the sign carried into the final scale of dK.
    u32x4 kf[NC], vf[NC];
#pragma unroll
    for (int dc = 0; dc < NC; ++dc) {
        kf[dc] = load16(rk, (uint32_t)((myk * kD + 16 * dc + 8 * h) * 2));
        vf[dc] = load16(rv, (uint32_t)((myk * kD + 16 * dc + 8 * h) * 2)) ^ 0x80008000u;
    }
    const bool klive = myk < Nk;

    // queries this key block sees: causal starts at the tile holding key k0
    const int qstart = CAUSAL ? (k0 / kBlk) * kBlk : 0;
    const int ntile = qstart < Nq ? (Nq - qstart + kBlk - 1) / kBlk : 0;
    const TileOfs<D, 2> to(lane, dbase);

    if (Nq % kBlk != 0) {  // rows past Nq are never loaded: keep them finite
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < D / 16; ++i) {
            reinterpret_cast<u32x4 *>(sQ)[tid + 256 * i] = z;
            reinterpret_cast<u32x4 *>(sG)[tid + 256 * i] = z;
        }
        if (tid < 64) reinterpret_cast<u32x4 *>(sL)[tid] = z;
        __syncthreads();
    }

    // L and D of 64 query rows into sl[0, 64) and sl[64, 128): lanes 0-15 of
    // wave 0 move 16 bytes (4 rows) each, once from each tensor.
    auto dma_ld = [&](float *sl, int r0) {
        if (wave == 0 && lane < 16) {
            const uint32_t off = (uint32_t)((r0 + 4 * lane) * 4);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_void *)sl, 16, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_void *)(sl + kBlk), 16, off, 0, 0, 0);
        }
    };

    f32x16 dk[2], dv[2];  // dK^T / dV^T: [dt][r] = X[myk][dbase + 32dt + 8(r/4) + 4h + r%4]
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[0][i] = dk[1][i] = dv[0][i] = dv[1][i] = 0.f;

    // S and D - dP of one 32-query sub-tile (rows qt / gt of the staged tile,
    // L and D in sl): s[r], dn[r] belong to query qa + 8(r/4) + 4h + r%4 and
    // key myk.  The second product starts from the staged D (four
    // consecutive rows per 16-byte read land in four accumulator registers).
    auto prod = [&](int qa, const uint16_t *qt, const uint16_t *gt, const float *sl, f32x16 &s,
                    f32x16 &dn) {
        const int tb = (qa & (kBlk - 1)) + 4 * h;  // staged row of r = 0
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 d4 = *reinterpret_cast<const f32x4 *>(sl + kBlk + tb + 8 * g4);
#pragma unroll
            for (int i = 0; i < 4; ++i) dn[4 * g4 + i] = d4[i];
        }
#pragma unroll
        for (int dc = 0; dc < NC; ++dc) {
            s = mma<DT>(read_row(qt, to.row_ofs[dc]), kf[dc], dc == 0 ? f32x16{} : s);
            dn = mma<DT>(read_row(gt, to.row_ofs[dc]), vf[dc], dn);
        }
    };
    // P = exp2(c S - L log2 e) and -dS = P o (D - dP), rounded and packed as
    // the B operands of dV^T and dK^T.  The staged L is already in base-2
    // units, +inf on rows past Nq (P = 0 there without a test).  With MASK,
    // queries before the key get P = 0 (causal).
    auto softgrad = [&](auto mask_tag, int qa, const float *sl, const f32x16 &s, const f32x16 &dn,
                        u32x4 *pp, u32x4 *pd) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int tb = (qa & (kBlk - 1)) + 4 * h;
        f32x4 lq[4];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) lq[g4] = *reinterpret_cast<const f32x4 *>(sl + tb + 8 * g4);
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float pv[2], dsv[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int r = 8 * c + 2 * j + e;
                    float x = __builtin_fmaf(s[r], scale_log2, -lq[r >> 2][r & 3]);
                    if constexpr (MASK) {
                        const int q = qa + 8 * (r >> 2) + 4 * h + (r & 3);
                        x = myk <= q ? x : -INFINITY;
                    }
                    pv[e] = exp2f_fast(x);
                    dsv[e] = pv[e] * dn[r];
                }
                pp[c][j] = pack2<DT>(pv[0], pv[1]);
                pd[c][j] = pack2<DT>(dsv[0], dsv[1]);
            }
    };
    // dV^T += dO^T P and dK^T += Q^T dS (contraction over the 32 queries;
    // dO^T and Q^T by the transposed read of the staged rows)
    auto grad = [&](const uint16_t *qt, const uint16_t *gt, const u32x4 *pp, const u32x4 *pd) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int dt = 0; dt < 2; ++dt) {
                dv[dt] = mma<DT>(read_tr<D>(gt, to.tr_ofs[dt], c), pp[c], dv[dt]);
                dk[dt] = mma<DT>(read_tr<D>(qt, to.tr_ofs[dt], c), pd[c], dk[dt]);
            }
    };
    // One staged 64-query tile: sub-tiles A (rows r0..r0+31) and B.  With
    // causal masking A may lie wholly before this wave's keys (then only B
    // runs).  B's products are issued before A's exponentials and A's
    // gradient products before B's, so the matrix cores have work while the
    // vector ALUs run.
    auto compute = [&](auto mask_tag, int r0, const uint16_t *qc, const uint16_t *gc, const float *slc,
                       bool doA) {
        f32x16 sA, dA, sB, dB;
        u32x4 pA[2], qA[2], pB[2], qB[2];
        const uint16_t *qb = qc + 32 * kD, *gb = gc + 32 * kD;
        if (doA) prod(r0, qc, gc, slc, sA, dA);
        if (FA2_BWD_PIPE_KV) prod(r0 + 32, qb, gb, slc, sB, dB);
        if (doA) {
            softgrad(mask_tag, r0, slc, sA, dA, pA, qA);
            grad(qc, gc, pA, qA);
        }
        __builtin_amdgcn_sched_barrier(0);  // as in the dQ kernel
        if (!FA2_BWD_PIPE_KV) prod(r0 + 32, qb, gb, slc, sB, dB);
        softgrad(mask_tag, r0 + 32, slc, sB, dB, pB, qB);
        grad(qb, gb, pB, qB);
    };

    auto stage = [&](int t, uint16_t *qd, uint16_t *gd, float *sld) {
        const int r0 = qstart + t * kBlk;
        dma_tile<D>(rq, qd, r0, wave, lane);
        dma_tile<D>(rdo, gd, r0, wave, lane);
        dma_ld(sld, r0);
    };
    // After wave 0's copy of tile t's L has landed (its own wait), L goes to
    // base-2 units and rows past Nq get L = +inf: their P is then exp2(-inf)
    // = 0 and dS = 0.  The barrier that follows publishes the writes.
    auto seal = [&](int t, float *sl) {
        const int r0 = qstart + t * kBlk;
        if (wave == 0) sl[lane] = r0 + lane < Nq ? sl[lane] * kLog2e : INFINITY;
    };
    if (ntile > 0) {
        stage(0, sQ, sG, sL);
        __builtin_amdgcn_s_waitcnt(0);
        seal(0, sL);
        __syncthreads();
    }
    auto tile = [&](auto mask_tag, int t, const uint16_t *qc, const uint16_t *gc, const float *slc,
                    uint16_t *qd, uint16_t *gd, float *sld) {
        constexpr bool MASK = decltype(mask_tag)::value;
        if (t + 1 < ntile) stage(t + 1, qd, gd, sld);
        const int r0 = qstart + t * kBlk;
        if constexpr (MASK) {  // some query of the tile is before some key (causal)
            const bool doA = r0 + 31 >= kw;
            const bool doB = r0 + 63 >= kw;
            if (doB) compute(std::true_type{}, r0, qc, gc, slc, doA);
        } else {
            compute(std::false_type{}, r0, qc, gc, slc, true);
        }
        __builtin_amdgcn_s_waitcnt(0);
        if (t + 1 < ntile) seal(t + 1, sld);
        __syncthreads();
    };
    // Causal: the tiles on this wave's diagonal (a query before one of its
    // keys) come first and take the masked path in a loop of their own; the
    // rest run unmasked in a second loop (one copy of the tile per loop keeps
    // the accumulators in place).  Each wave still passes one barrier per tile.
    const int tm = CAUSAL ? min(ntile, (kw + 31 - qstart + kBlk - 1) / kBlk) : 0;
    int t = 0;
    for (; t < tm; ++t) {
        const int cur = (t & 1) * kBlk * kD, nxt = kBlk * kD - cur;
        const int lcur = (t & 1) * 2 * kBlk, lnxt = 2 * kBlk - lcur;
        tile(std::true_type{}, t, sQ + cur, sG + cur, sL + lcur, sQ + nxt, sG + nxt, sL + lnxt);
    }
    for (; t < ntile; ++t) {
        const int cur = (t & 1) * kBlk * kD, nxt = kBlk * kD - cur;
        const int lcur = (t & 1) * 2 * kBlk, lnxt = 2 * kBlk - lcur;
        tile(std::false_type{}, t, sQ + cur, sG + cur, sL + lcur, sQ + nxt, sG + nxt, sL + lnxt);
    }

    if (klive) {
        const float nscale = -scale;  // the accumulated dS had its sign flipped
        uint16_t *krow = dK + ((size_t)bh * Nk + myk) * kD;
        uint16_t *vrow = dV + ((size_t)bh * Nk + myk) * kD;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int r = 4 * g4;
                const int d = dbase + 32 * dt + 8 * g4 + 4 * h;
                u32x2 w;
                w[0] = pack2<DT>(dk[dt][r] * nscale, dk[dt][r + 1] * nscale);
                w[1] = pack2<DT>(dk[dt][r + 2] * nscale, dk[dt][r + 3] * nscale);
                *reinterpret_cast<u32x2 *>(krow + d) = w;
                w[0] = pack2<DT>(dv[dt][r], dv[dt][r + 1]);
                w[1] = pack2<DT>(dv[dt][r + 2], dv[dt][r + 3]);
                *reinterpret_cast<u32x2 *>(vrow + d) = w;
            }
    }
}

template <int D, int DT>
fa2_status bwd_dt(const BwdArgs &a, hipStream_t st) {
    const int bh = a.B * a.H;
    const uint16_t *q = (const uint16_t *)a.q, *k = (const uint16_t *)a.k, *v = (const uint16_t *)a.v;
    const uint16_t *o = (const uint16_t *)a.o, *g = (const uint16_t *)a.dout;
    const float sl2 = a.scale * kLog2e;
    fa2_status s = FA2_OK;
    if (a.Nq > 0) {
        constexpr int rows_per_wg = 256 / (D / 8);  // delta kernel: D/8 lanes per row
        s = launch(bwd_delta_kernel<D, DT>, dim3((a.Nq + rows_per_wg - 1) / rows_per_wg, bh), dim3(256),
                   st, o, g, a.delta, a.Nq);
        if (s != FA2_OK) return s;
        auto kq = a.causal ? bwd_dq_kernel<D, DT, true> : bwd_dq_kernel<D, DT, false>;
        s = launch(kq, dim3((unsigned)((a.Nq + kRows - 1) / kRows) * bh), dim3(kWaves * 64), st, q, k, v,
                   g, a.lse, (const float *)a.delta, (uint16_t *)a.dq, bh, a.Nq, a.Nk, a.scale, sl2);
        if (s != FA2_OK) return s;
    }
    // with no queries this still runs: it writes dK = dV = 0
    constexpr int kpw = kv_keys_per_wg<D>();
    auto kk = a.causal ? bwd_dkdv_kernel<D, DT, true> : bwd_dkdv_kernel<D, DT, false>;
    return launch(kk, dim3((unsigned)((a.Nk + kpw - 1) / kpw) * bh), dim3(kWaves * 64), st, q, k, v, g,
                  a.lse, (const float *)a.delta, (uint16_t *)a.dk, (uint16_t *)a.dv, bh, a.Nq, a.Nk,
                  a.scale, sl2);
}

}  // namespace

fa2_status launch_bwd_mfma(const BwdArgs &a, fa2_dtype dt, hipStream_t st) {
    if (a.D == 128) return dt == FA2_F16 ? bwd_dt<128, 1>(a, st) : bwd_dt<128, 2>(a, st);
    return dt == FA2_F16 ? bwd_dt<64, 1>(a, st) : bwd_dt<64, 2>(a, st);
}

}  // namespace fa2
