// fwd_f32.hip -- exact attention forward, float32 in and out, D = 64, on the
// float32 matrix cores of gfx950 (v_mfma_f32_16x16x4_f32: full f32 operands,
// f32 accumulation; nothing is rounded to a narrower type).
//
// Method ("Flash attention, f32": sections One block of queries per CTA, The
// loop over keys, Online softmax, After the loop; "Flash Attention"
// (aarnphm.xyz): Deriving the online softmax, tile form).  A workgroup owns 16
// query rows.  Its 8 waves each walk a contiguous slice of the keys, 16 keys a
// step, carrying the running max m, the running denominator l and the
// unnormalised output O, rescaled by exp(m_old - m_new) whenever the max grows.
// At the end the 8 partial states are merged with the (m, l) monoid of "Flash
// Attention" (section Deriving the online softmax) through LDS, then O/l and
// LSE = m + ln l are written.
//
// Why split the keys across waves: one head of 4096 rows gives only 256 tiles
// of 16 rows, one per compute unit; splitting each tile's keys 8 ways puts two
// waves on every SIMD.  The pages' FlashAttention-2 prefers splitting queries
// across warps ("Flash Attention", section FlashAttention 2); this kernel keeps
// that across workgroups and splits keys only inside one.
//
// Lane layout (lane = 16*g + c):
//   S^T = K Q^T per 16-key step: lane holds scores of query c for keys 4g..4g+3.
//   O^T = V^T P^T: lane holds O[query c][16g .. 16g+15] (the MFMA's n index is
//   permuted so that each lane's V operand is one 16-byte row segment).
// The contraction index of both products is only a pairing of operand slots,
// so A and B just have to agree on it.
#include "fa2_device.h"
#include "fa2_internal.h"

namespace fa2 {

namespace {

constexpr int kD = 64;
constexpr int kQT = 16;     // query rows per workgroup
constexpr int kWaves = 8;   // waves per workgroup, each on its own key slice
constexpr int kStep = 16;   // keys per step

struct KVRegs {
    f32x4 k[4];   // K[key k0 + c][16g .. 16g+15]
    f32x4 v[4];   // V[key k0 + 4g + t][4c .. 4c+3], t = 0..3
};

__device__ __forceinline__ void load_kv(KVRegs &r, __amdgpu_buffer_rsrc_t rk,
                                        __amdgpu_buffer_rsrc_t rv, int k0, int g, int c) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
        r.k[j] = __builtin_bit_cast(f32x4, load16(rk, (uint32_t)(((k0 + c) * kD + 16 * g + 4 * j) * 4)));
#pragma unroll
    for (int t = 0; t < 4; ++t)
        r.v[t] = __builtin_bit_cast(f32x4, load16(rv, (uint32_t)(((k0 + 4 * g + t) * kD + 4 * c) * 4)));
}

template <bool CAUSAL>
__global__ __launch_bounds__(kWaves * 64, 1) void fwd_f32_d64_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    float *__restrict__ O, float *__restrict__ LSE, int Nq, int Nk, float scale_log2) {
    __shared__ __attribute__((aligned(16))) float s_o[kWaves][kQT][kD];
    __shared__ float s_m[kWaves][kQT];
    __shared__ float s_l[kWaves][kQT];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int q0 = blockIdx.x * kQT;
    const int bh = blockIdx.y;

    const float *Qh = Q + (size_t)bh * Nq * kD;
    const float *Kh = K + (size_t)bh * Nk * kD;
    const float *Vh = V + (size_t)bh * Nk * kD;
    const auto rq = make_rsrc(Qh, (uint32_t)Nq * kD * 4);
    const auto rk = make_rsrc(Kh, (uint32_t)Nk * kD * 4);
    const auto rv = make_rsrc(Vh, (uint32_t)Nk * kD * 4);

    // Q^T operand of S^T = K Q^T: slot i of lane (g,c) is Q[q0 + c][16g + i].
    float qv[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f32x4 t = __builtin_bit_cast(f32x4, load16(rq, (uint32_t)(((q0 + c) * kD + 16 * g + 4 * j) * 4)));
        qv[4 * j + 0] = t[0];
        qv[4 * j + 1] = t[1];
        qv[4 * j + 2] = t[2];
        qv[4 * j + 3] = t[3];
    }

    const int kend = CAUSAL ? min(Nk, q0 + kQT) : Nk;
    const int nsteps = (kend + kStep - 1) / kStep;
    const int per = (nsteps + kWaves - 1) / kWaves;
    const int st0 = wave * per;
    const int st1 = min(nsteps, st0 + per);

    float m = -INFINITY;  // running max of scaled scores, base-2 units
    float l = 0.f;        // this lane's share of the running denominator
    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    KVRegs cur, nxt;
    if (st0 < st1) load_kv(cur, rk, rv, st0 * kStep, g, c);
    for (int st = st0; st < st1; ++st) {
        const int k0 = st * kStep;
        if (st + 1 < st1) load_kv(nxt, rk, rv, k0 + kStep, g, c);

        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 16; ++i)
            sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(cur.k[i >> 2][i & 3], qv[i], sacc, 0, 0, 0);

        // sacc[r] = S[query q0 + c][key k0 + 4g + r]
        float s[4];
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = k0 + 4 * g + r;
            bool live = key < Nk;
            if (CAUSAL) live = live && key <= q0 + c;
            s[r] = live ? sacc[r] * scale_log2 : -INFINITY;
            mx = fmaxf(mx, s[r]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float corr = exp2f_fast(m - m_use);
        float p[4];
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p[r] = exp2f_fast(s[r] - m_use);
            psum += p[r];
        }
        l = l * corr + psum;
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] *= corr;
        // O^T += V^T P^T: slot g pairs key k0 + 4g + t; row m of tile j is d = 4m + j.
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(cur.v[t][j], p[t], acc[j], 0, 0, 0);
        m = m_new;
        if (st + 1 < st1) cur = nxt;
    }

    // acc[j][r] = O[q0 + c][16g + 4r + j]; the lane's l covers keys 4g..4g+3 of each step.
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (g == 0) {
        s_m[wave][c] = m;
        s_l[wave][c] = l;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
        *reinterpret_cast<f32x4 *>(&s_o[wave][c][16 * g + 4 * r]) =
            f32x4{acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
    __syncthreads();

    // Merge the 8 wave states of each row: 512 threads, 2 output columns each.
    const int row = threadIdx.x >> 5;
    const int d = (threadIdx.x & 31) * 2;
    float mg = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mg = fmaxf(mg, s_m[w][row]);
    float lg = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const float mw = s_m[w][row];
        const float wt = mw == -INFINITY ? 0.f : exp2f_fast(mw - mg);
        lg += wt * s_l[w][row];
        o0 += wt * s_o[w][row][d];
        o1 += wt * s_o[w][row][d + 1];
    }
    const int qrow = q0 + row;
    if (qrow < Nq) {
        const float inv = 1.f / lg;
        float *orow = O + ((size_t)bh * Nq + qrow) * kD;
        orow[d] = o0 * inv;
        orow[d + 1] = o1 * inv;
        if (LSE && d == 0) LSE[(size_t)bh * Nq + qrow] = (mg + log2f_fast(lg)) * kLn2;
    }
}

}  // namespace

fa2_status launch_fwd_f32_d64(const FwdArgs &a, hipStream_t st) {
    const dim3 grid((a.Nq + kQT - 1) / kQT, a.B * a.H);
    const dim3 block(kWaves * 64);
    const float sl2 = a.scale * kLog2e;
    if (a.causal)
        return launch(fwd_f32_d64_kernel<true>, grid, block, st, (const float *)a.q,
                      (const float *)a.k, (const float *)a.v, (float *)a.o, a.lse, a.Nq, a.Nk,
                      sl2);
    return launch(fwd_f32_d64_kernel<false>, grid, block, st, (const float *)a.q,
                  (const float *)a.k, (const float *)a.v, (float *)a.o, a.lse, a.Nq, a.Nk, sl2);
}

}  // namespace fa2
