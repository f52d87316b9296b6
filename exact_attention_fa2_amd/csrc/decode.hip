// decode.hip -- flash-decoding on gfx950: one query row per (batch, head)
// against a long K/V cache, split along the sequence ("Flash decoding":
// Overview of the algorithm, the split kernel and the combine kernel).
//
// Split kernel: one workgroup per (split, b*h).  The step is bound by HBM
// reads of K and V, not by arithmetic (one multiply-add per loaded element),
// so the scores are a GEMV on the vector ALUs and the design goal is bytes in
// flight: every lane issues 8 independent 16-byte loads of K and 8 of V per
// step, each wave covering 8*R keys (R rows per wave-wide load: 4 for a
// 256-byte row).  The CH lanes that share a row each hold one 16-byte chunk of
// q, K_j and V_j; the dot product is reduced over those lanes with DPP.  Each
// row group keeps its own online-softmax state (m, l, O chunk), and the
// workgroup merges its 4 waves x R row groups with the (m, l) monoid in LDS
// before writing one unnormalised partial (O_s, m_s, l_s).
//
// Combine kernel: one output row per (b,h), four output columns per thread
// and several rows per workgroup; weights exp(m_s - m_g), a single division
// by l_g at the end.  It also merges the key-split partials of the forward
// kernels (one output row per query row); those may carry a second
// denominator for the LSE.
#include "fa2_device.h"
#include "fa2_internal.h"

namespace fa2 {

namespace {

// Tuning knobs: 16-byte loads per lane per step for each of K and V, and the
// cache-policy bits of those loads: 2 marks them non-temporal (K and V are
// read exactly once), which measured 6.1 -> 7.0 TB/s on the decode workload.
#ifndef FA2_DEC_UNROLL
#define FA2_DEC_UNROLL 8
#endif
#ifndef FA2_DEC_AUX
#define FA2_DEC_AUX 2
#endif

constexpr int kWaves = 4;
constexpr int kUnroll = FA2_DEC_UNROLL;

template <int DT>
struct Elem {
    static constexpr int size = DT == 0 ? 4 : 2;
};

// The EPC values in one 16-byte chunk, as floats.
template <int DT>
__device__ __forceinline__ void to_float(u32x4 w, float *out) {
    if constexpr (DT == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(w[i]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) unpack2<DT>(w[i], out[2 * i], out[2 * i + 1]);
    }
}

template <int DT>
__device__ __forceinline__ float chunk_dot(u32x4 qw, const float *qf, u32x4 kw) {
    if constexpr (DT == 0) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) s = __builtin_fmaf(qf[i], __uint_as_float(kw[i]), s);
        return s;
    } else {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) s = dot2<DT>(qw[i], kw[i], s);
        return s;
    }
}

template <int DT, int D>
__global__ __launch_bounds__(kWaves * 64) void decode_split_kernel(
    const void *__restrict__ Q, const void *__restrict__ K, const void *__restrict__ V,
    float *__restrict__ o_part, float *__restrict__ m_part, float *__restrict__ l_part, int N,
    int n_splits, int S, float scale_log2) {
    constexpr int ESZ = Elem<DT>::size;
    constexpr int CH = D * ESZ / 16;  // lanes per row
    constexpr int R = 64 / CH;        // rows per wave-wide load
    constexpr int EPC = 16 / ESZ;     // elements per 16-byte chunk
    constexpr int KPS = kUnroll * R;  // keys per wave step
    static_assert(CH == 8 || CH == 16 || CH == 32, "row width");

    __shared__ float s_m[kWaves * R], s_l[kWaves * R];
    __shared__ __attribute__((aligned(16))) float s_o[kWaves * R][D];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rg = lane / CH, c = lane % CH;
    const int sp = blockIdx.x;
    const int bh = blockIdx.y;
    const int n0 = sp * S;
    const int n1 = min(n0 + S, N);

    const size_t head = (size_t)bh * N * D * ESZ;
    const auto rk = make_rsrc((const char *)K + head, (uint32_t)N * D * ESZ);
    const auto rv = make_rsrc((const char *)V + head, (uint32_t)N * D * ESZ);
    const auto rq = make_rsrc((const char *)Q + (size_t)bh * D * ESZ, (uint32_t)D * ESZ);

    const u32x4 qw = load16(rq, (uint32_t)(c * 16));
    float qf[EPC];
    to_float<DT>(qw, qf);

    float m = -INFINITY, l = 0.f;
    float acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.f;

    for (int base = n0 + wave * KPS; base < n1; base += kWaves * KPS) {
        u32x4 kr[kUnroll], vr[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t off = (uint32_t)((base + u * R + rg) * (D * ESZ) + c * 16);
            kr[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)off, 0, FA2_DEC_AUX);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t off = (uint32_t)((base + u * R + rg) * (D * ESZ) + c * 16);
            vr[u] = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)off, 0, FA2_DEC_AUX);
        }
        float sc[kUnroll];
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const float dot = group_reduce<CH>(chunk_dot<DT>(qw, qf, kr[u]));
            const bool live = base + u * R + rg < n1;
            sc[u] = live ? dot * scale_log2 : -INFINITY;
            mx = fmaxf(mx, sc[u]);
        }
        const float m_new = fmaxf(m, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float corr = exp2f_fast(m - m_use);
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[e] *= corr;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const float p = exp2f_fast(sc[u] - m_use);
            psum += p;
            float vf[EPC];
            to_float<DT>(vr[u], vf);
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[e] = __builtin_fmaf(p, vf[e], acc[e]);
        }
        l = l * corr + psum;
        m = m_new;
    }

    const int slot = wave * R + rg;
    if (c == 0) {
        s_m[slot] = m;
        s_l[slot] = l;
    }
#pragma unroll
    for (int e = 0; e < EPC; ++e) s_o[slot][c * EPC + e] = acc[e];
    __syncthreads();

    for (int d = threadIdx.x; d < D; d += kWaves * 64) {
        float mg = -INFINITY;
        for (int i = 0; i < kWaves * R; ++i) mg = fmaxf(mg, s_m[i]);
        float lg = 0.f, o = 0.f;
        for (int i = 0; i < kWaves * R; ++i) {
            const float wt = s_m[i] == -INFINITY ? 0.f : exp2f_fast(s_m[i] - mg);
            lg += wt * s_l[i];
            o += wt * s_o[i][d];
        }
        const size_t pidx = (size_t)bh * n_splits + sp;
        o_part[pidx * D + d] = o;
        if (d == 0) {
            m_part[pidx] = mg == -INFINITY ? -INFINITY : mg * kLn2;  // natural-log units
            l_part[pidx] = lg;
        }
    }
}

// CPT output columns per thread (1 or 4), D/CPT threads per row, and
// blockDim.x / (D/CPT) rows per workgroup.  Many rows (the forward's
// key-split partials of tens of thousands of rows) take four columns per
// thread and up to 256 threads per workgroup: one single-wave workgroup per
// row left those bound by workgroup dispatch.  Few rows (decode, few-tile
// splits) take one row per workgroup and one column per thread, which keeps
// more loads in flight per row.
template <int CPT>
struct Cols;
template <>
struct Cols<1> {
    typedef float type;
};
template <>
struct Cols<4> {
    typedef f32x4 type;
};

template <int DT, int D, int CPT>
__global__ __launch_bounds__(256) void decode_combine_kernel(const float *__restrict__ o_part,
                                                             const float *__restrict__ m_part,
                                                             const float *__restrict__ l_part,
                                                             const float *__restrict__ l2_part,
                                                             void *__restrict__ O,
                                                             float *__restrict__ LSE, size_t rows,
                                                             int n_splits) {
    typedef typename Cols<CPT>::type vec;
    constexpr int TPR = D / CPT;
    // output row ((b,h) for decode); with one row per workgroup it is
    // wave-uniform, and the row's m and l come through scalar loads
    const size_t bh = CPT == 1 ? (size_t)blockIdx.x
                               : (size_t)blockIdx.x * (blockDim.x / TPR) + threadIdx.x / TPR;
    const int d = CPT * (threadIdx.x % TPR);
    if (bh >= rows) return;
    const float *mp = m_part + bh * n_splits;
    const float *lp = l_part + bh * n_splits;
    const float *op = o_part + bh * n_splits * D + d;
    float mg = -INFINITY;
#pragma unroll 8
    for (int s = 0; s < n_splits; ++s) mg = fmaxf(mg, mp[s]);
    float lg = 0.f, lg2 = 0.f;
    vec acc = {};
#pragma unroll 8
    for (int s = 0; s < n_splits; ++s) {
        const float ms = mp[s];
        const float wt = ms == -INFINITY ? 0.f : exp2f_fast((ms - mg) * kLog2e);
        lg += wt * lp[s];
        if (l2_part) lg2 += wt * l2_part[bh * n_splits + s];
        acc += wt * *reinterpret_cast<const vec *>(op + (size_t)s * D);
    }
    const vec o = acc / lg;
    if constexpr (DT == 0) {
        *reinterpret_cast<vec *>((float *)O + bh * D + d) = o;
    } else if constexpr (CPT == 1) {
        ((uint16_t *)O)[bh * D + d] = (uint16_t)(pack2<DT>(o, 0.f) & 0xFFFF);
    } else {
        const u32x2 w = {pack2<DT>(o[0], o[1]), pack2<DT>(o[2], o[3])};
        *reinterpret_cast<u32x2 *>((uint16_t *)O + bh * D + d) = w;
    }
    if (LSE && d == 0) LSE[bh] = mg + log2f_fast(l2_part ? lg2 : lg) * kLn2;
}

template <int DT, int D>
fa2_status split_dt(const DecodeArgs &a, hipStream_t st) {
    const int S = (int)(((long long)a.N + a.n_splits - 1) / a.n_splits);
    const dim3 grid(a.n_splits, a.B * a.H);
    return launch(decode_split_kernel<DT, D>, grid, dim3(kWaves * 64), st, a.q, a.k, a.v,
                  a.o_part, a.m_part, a.l_part, a.N, a.n_splits, S, a.scale * kLog2e);
}

template <int DT>
fa2_status combine_dt(const float *op, const float *mp, const float *lp, const float *lp2, void *o,
                      float *lse, size_t rows, int D, int ns, hipStream_t st) {
    if (rows > 0x7FFFFFFF) return FA2_ERR_UNSUPPORTED;
    if (rows * D < (size_t)1 << 20) {  // one row per workgroup, one column per thread
        if (D == 64)
            return launch(decode_combine_kernel<DT, 64, 1>, dim3((unsigned)rows), dim3(64), st, op, mp,
                          lp, lp2, o, lse, rows, ns);
        return launch(decode_combine_kernel<DT, 128, 1>, dim3((unsigned)rows), dim3(128), st, op, mp, lp,
                      lp2, o, lse, rows, ns);
    }
    // four columns per thread, 256 threads: 16 (D = 64) or 8 (D = 128) rows
    if (D == 64)
        return launch(decode_combine_kernel<DT, 64, 4>, dim3((unsigned)((rows + 15) / 16)), dim3(256), st,
                      op, mp, lp, lp2, o, lse, rows, ns);
    return launch(decode_combine_kernel<DT, 128, 4>, dim3((unsigned)((rows + 7) / 8)), dim3(256), st, op,
                  mp, lp, lp2, o, lse, rows, ns);
}

}  // namespace

fa2_status launch_decode_split(const DecodeArgs &a, fa2_dtype dt, hipStream_t st) {
    if (a.D == 64) {
        if (dt == FA2_F32) return split_dt<0, 64>(a, st);
        if (dt == FA2_F16) return split_dt<1, 64>(a, st);
        return split_dt<2, 64>(a, st);
    }
    if (dt == FA2_F32) return split_dt<0, 128>(a, st);
    if (dt == FA2_F16) return split_dt<1, 128>(a, st);
    return split_dt<2, 128>(a, st);
}

fa2_status launch_combine_rows(const float *o_part, const float *m_part, const float *l_part,
                               void *o, float *lse, size_t rows, int D, int n_splits, fa2_dtype dt,
                               hipStream_t st, const float *l2_part) {
    if (dt == FA2_F32)
        return combine_dt<0>(o_part, m_part, l_part, l2_part, o, lse, rows, D, n_splits, st);
    if (dt == FA2_F16)
        return combine_dt<1>(o_part, m_part, l_part, l2_part, o, lse, rows, D, n_splits, st);
    return combine_dt<2>(o_part, m_part, l_part, l2_part, o, lse, rows, D, n_splits, st);
}

fa2_status launch_decode_combine(const float *o_part, const float *m_part, const float *l_part,
                                 void *o, int B, int H, int D, int n_splits, fa2_dtype dt,
                                 hipStream_t st) {
    return launch_combine_rows(o_part, m_part, l_part, o, nullptr, (size_t)B * H, D, n_splits, dt,
                               st);
}

}  // namespace fa2
