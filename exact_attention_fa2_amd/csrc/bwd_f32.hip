// bwd_f32.hip -- exact attention backward, float32 in and out, D = 64 or 128,
// on the float32 matrix cores of gfx950 (v_mfma_f32_16x16x4_f32: full f32
// operands, f32 accumulation; nothing is rounded to a narrower type).
//
// Method, as in bwd.hip ("Flash Attention" (aarnphm.xyz), section IO
// complexity, the paragraph on the backward pass; "06: Fused attention", the
// backward kernels): only O and the per-row log-sum-exp L are kept from the
// forward, and with D_i = rowsum(dO o O)
//     P = exp(scale S - L),  dP = dO V^T,  dS = P o (dP - D_i),
//     dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K.
// Three kernels: D (one pass over O and dO); dQ (a workgroup per 16 query
// rows whose 8 waves each walk a contiguous slice of the keys); dK/dV (a
// workgroup per 16 keys whose waves walk slices of the queries; at D = 128
// two waves share each slice and keep one 64-column half of dK and dV each).
// The waves' partial sums are added through LDS at the end, so nothing is
// accumulated with atomics and the results do not depend on timing.
//
// Lane layout (lane = 16*g + c), as in the float32 forward: the 16x16x4 MFMA
// leaves rows 4g..4g+3 of column c in lane (g, c), and the contraction index
// is only a pairing of operand slots, so A and B just have to agree on it.
//   dQ kernel (column = query c):  S^T = K Q^T and dP^T = V dO^T pair
//     d = 16(i/4) + 4g + i%4 in MFMA i; dQ^T += K^T dS^T takes the lane's own
//     four dS values (keys 4g..4g+3) as its B operand.
//   dK/dV kernel (column = key c):  S = Q K^T, dP = dO V^T, then
//     dV^T += dO^T P and dK^T += Q^T dS with the lane's own P and dS.
// Row m of output tile 4h + j is column 64h + 4m + j of the [.., D] tensor,
// so each lane reads the A operands of the second products as 16-byte row
// pieces.
#include "fa2_device.h"
#include "fa2_internal.h"

namespace fa2 {

namespace {

constexpr int kT = 16;     // rows of a workgroup's tile (queries, or keys)
constexpr int kW = 8;      // waves per workgroup (2 per SIMD)
constexpr int kStep = 16;  // keys (dQ) or queries (dK/dV) per step

// Tile and head of this workgroup in a one-dimensional grid with b*h varying
// fastest (workgroups that arrive together have the same length under a
// causal mask); `rev` hands out the tiles from the last one.
__device__ __forceinline__ void tile_head(int n_tiles, bool rev, int &t, int &bh) {
    const int n_bh = gridDim.x / n_tiles;
    const int rank = blockIdx.x / n_bh;
    bh = blockIdx.x - rank * n_bh;
    t = rev ? n_tiles - 1 - rank : rank;
}

// A operands: N 16-byte pieces per lane.  Rows past the descriptor's range
// read as 0.
template <int N>
struct Op {
    f32x4 x[N];
};

// Rows r0..r0+15 of a tensor with rows of `ld` floats, by rows (first
// products), N pieces from column col0 on:
//   x[j] = X[r0 + c][col0 + 16j + 4g .. col0 + 16j + 4g + 3]
template <int N>
__device__ __forceinline__ void load_rows(Op<N> &o, __amdgpu_buffer_rsrc_t r, int r0, int ld,
                                          int col0, int g, int c) {
#pragma unroll
    for (int j = 0; j < N; ++j)
        o.x[j] = __builtin_bit_cast(f32x4, load16(r, (uint32_t)(((r0 + c) * ld + col0 + 16 * j + 4 * g) * 4)));
}

// ... and by columns (second products), the 64 columns from col0 on:
//   x[t] = X[r0 + 4g + t][col0 + 4c .. col0 + 4c + 3]
__device__ __forceinline__ void load_cols(Op<4> &o, __amdgpu_buffer_rsrc_t r, int r0, int ld,
                                          int col0, int g, int c) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
        o.x[t] = __builtin_bit_cast(f32x4, load16(r, (uint32_t)(((r0 + 4 * g + t) * ld + col0 + 4 * c) * 4)));
}

// B operand slots of row `row`, 16N columns from col0 on:
//   v[i] = X[row][col0 + 16(i/4) + 4g + i%4]
template <int N>
__device__ __forceinline__ void load_bop(float *v, __amdgpu_buffer_rsrc_t r, int row, int ld,
                                         int col0, int g) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const f32x4 t = __builtin_bit_cast(f32x4, load16(r, (uint32_t)((row * ld + col0 + 16 * j + 4 * g) * 4)));
        v[4 * j + 0] = t[0];
        v[4 * j + 1] = t[1];
        v[4 * j + 2] = t[2];
        v[4 * j + 3] = t[3];
    }
}

__device__ __forceinline__ f32x4 mfma(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// sum_i A_i B_i over the 4N pairings of a 16N-long contraction, in two chains
template <int N>
__device__ __forceinline__ f32x4 product(const Op<N> &a, const float *b) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f}, s2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4 * N; i += 2) {
        s = mfma(a.x[i >> 2][i & 3], b[i], s);
        s2 = mfma(a.x[i >> 2][(i & 3) + 1], b[i + 1], s2);
    }
    return s + s2;
}

// acc[j] += X^T W: tile j of a [64 x 16] result, W slot t = the lane's own
// value for row 4g + t of the step.
__device__ __forceinline__ void accumulate(f32x4 *acc, const Op<4> &x, const float *w) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = mfma(x.x[t][j], w[t], acc[j]);
}

// D_i = sum_d dO_id O_id: 16 lanes per row (D/16 values each), 16 rows per
// workgroup.
template <int D>
__global__ __launch_bounds__(256) void bwd_f32_delta_kernel(const float *__restrict__ O,
                                                            const float *__restrict__ dO,
                                                            float *__restrict__ Delta, int Nq) {
    const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
    const int c = threadIdx.x & 15;
    const size_t base = (size_t)blockIdx.y * Nq;
    float acc = 0.f;
    if (row < Nq) {
#pragma unroll
        for (int h = 0; h < D / 64; ++h) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(O + (base + row) * D + 64 * h + 4 * c);
            const f32x4 b = *reinterpret_cast<const f32x4 *>(dO + (base + row) * D + 64 * h + 4 * c);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(a[i], b[i], acc);
        }
    }
    acc = group_reduce<16>(acc);
    if (row < Nq && c == 0) Delta[base + row] = acc;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kW * 64, 1) void bwd_f32_dq_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    const float *__restrict__ dO, const float *__restrict__ LSE, const float *__restrict__ Delta,
    float *__restrict__ dQ, int Nq, int Nk, float scale, float scale_log2) {
    constexpr int NH = D / 64;  // 64-column blocks of dQ, all kept by every wave
    __shared__ __attribute__((aligned(16))) float s_acc[kW][kT][D];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, c = lane & 15;
    int qt, bh;
    tile_head((Nq + kT - 1) / kT, CAUSAL, qt, bh);  // causal: the longest rows first
    const int q0 = qt * kT;
    const int myq = q0 + c;

    const auto rq = make_rsrc(Q + (size_t)bh * Nq * D, (uint32_t)Nq * D * 4);
    const auto rdo = make_rsrc(dO + (size_t)bh * Nq * D, (uint32_t)Nq * D * 4);
    const auto rk = make_rsrc(K + (size_t)bh * Nk * D, (uint32_t)Nk * D * 4);
    const auto rv = make_rsrc(V + (size_t)bh * Nk * D, (uint32_t)Nk * D * 4);

    float qv[D / 4], gv[D / 4];  // B operands: this lane's query row of Q and of dO
    load_bop<D / 16>(qv, rq, myq, D, 0, g);
    load_bop<D / 16>(gv, rdo, myq, D, 0, g);
    const bool qlive = myq < Nq;
    const float l2 = qlive ? LSE[(size_t)bh * Nq + myq] * kLog2e : 0.f;  // L in base 2
    const float dl = qlive ? Delta[(size_t)bh * Nq + myq] : 0.f;

    const int kend = CAUSAL ? min(Nk, q0 + kT) : Nk;
    const int nsteps = (kend + kStep - 1) / kStep;
    const int per = (nsteps + kW - 1) / kW;
    const int st0 = wave * per;
    const int st1 = min(nsteps, st0 + per);

    // acc[4h + j][r] = dQ[myq][64h + 16g + 4r + j] / scale over this wave's keys
    f32x4 acc[4 * NH];
#pragma unroll
    for (int j = 0; j < 4 * NH; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    struct Ops {
        Op<D / 16> k, v;  // K and V by rows (first products)
        Op<4> kc[NH];     // K by columns (dQ^T), per 64-column block
    };
    auto load = [&](Ops &o, int k0) {
        load_rows(o.k, rk, k0, D, 0, g, c);
        load_rows(o.v, rv, k0, D, 0, g, c);
#pragma unroll
        for (int h = 0; h < NH; ++h) load_cols(o.kc[h], rk, k0, D, 64 * h, g, c);
    };
    auto compute = [&](int st, const Ops &cur) {
        const int k0 = st * kStep;
        const f32x4 s = product(cur.k, qv);   // s[r]: S[myq][k0 + 4g + r]
        const f32x4 dp = product(cur.v, gv);  // dP, same slots
        const bool in_slice = st < st1;
        float ds[4];
        // the per-score mask only on steps that reach past Nk or Nq, cross the
        // diagonal or lie past this wave's slice (a wave-uniform test)
        if (in_slice && k0 + kStep <= Nk && q0 + kT <= Nq && !(CAUSAL && k0 + kStep - 1 > q0)) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ds[r] = exp2f_fast(__builtin_fmaf(s[r], scale_log2, -l2)) * (dp[r] - dl);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = k0 + 4 * g + r;
                bool live = in_slice && qlive && key < Nk;
                if (CAUSAL) live = live && key <= myq;
                const float p = live ? exp2f_fast(__builtin_fmaf(s[r], scale_log2, -l2)) : 0.f;
                ds[r] = p * (dp[r] - dl);
            }
        }
#pragma unroll
        for (int h = 0; h < NH; ++h) accumulate(acc + 4 * h, cur.kc[h], ds);
    };

    if constexpr (D == 64) {
        // One 16-key step on `cur`, with the next step's operands loaded into
        // `nxt` first (on every step, also past this wave's slice: in-range
        // data or zeros), so that the loads overlap this step's products.
        auto step = [&](int st, const Ops &cur, Ops &nxt) {
            load(nxt, (st + 1) * kStep);
            __builtin_amdgcn_sched_barrier(0);
            compute(st, cur);
        };
        Ops ra, rb;
        load(ra, st0 * kStep);
        for (int st = st0; st < st1; st += 2) {
            step(st, ra, rb);
            step(st + 1, rb, ra);
        }
    } else {
        // a second set of D = 128 operands does not fit the registers
        Ops cur;
        for (int st = st0; st < st1; ++st) {
            load(cur, st * kStep);
            compute(st, cur);
        }
    }

    // Add the waves' partial sums: one output element per thread and pass.
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            *reinterpret_cast<f32x4 *>(&s_acc[wave][c][64 * h + 16 * g + 4 * r]) =
                f32x4{acc[4 * h][r], acc[4 * h + 1][r], acc[4 * h + 2][r], acc[4 * h + 3][r]};
    __syncthreads();
    for (int e = threadIdx.x; e < kT * D; e += kW * 64) {
        const int row = e / D, d = e % D;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kW; ++w) sum += s_acc[w][row][d];
        if (q0 + row < Nq) dQ[((size_t)bh * Nq + q0 + row) * D + d] = sum * scale;
    }
}

// dK/dV.  At D = 128 the waves of a pair (2s, 2s + 1) walk the same queries:
// wave h forms the part of S and dP that columns 64h..64h+63 contribute, the
// pair adds its two parts through LDS, and each wave keeps dK and dV for its
// own 64 columns.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kW * 64, 1) void bwd_f32_dkdv_kernel(
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    const float *__restrict__ dO, const float *__restrict__ LSE, const float *__restrict__ Delta,
    float *__restrict__ dK, float *__restrict__ dV, int Nq, int Nk, float scale,
    float scale_log2) {
    constexpr int CS = D / 64;   // waves per query slice, one per 64 columns
    constexpr int NS = kW / CS;  // query slices
    __shared__ __attribute__((aligned(16))) float s_acc[2][NS][kT][D];
    // the pair's exchange of partial S and dP: [step parity][wave][S, dP][lane]
    __shared__ __attribute__((aligned(16))) f32x4 s_part[CS == 2 ? 2 : 1][CS == 2 ? kW : 1][2][64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slice = wave / CS, h = wave % CS;
    const int col0 = 64 * h;
    const int g = lane >> 4, c = lane & 15;
    int kt, bh;
    tile_head((Nk + kT - 1) / kT, false, kt, bh);  // causal: the first keys see the most queries
    const int k0 = kt * kT;
    const int myk = k0 + c;

    const auto rq = make_rsrc(Q + (size_t)bh * Nq * D, (uint32_t)Nq * D * 4);
    const auto rdo = make_rsrc(dO + (size_t)bh * Nq * D, (uint32_t)Nq * D * 4);
    const auto rk = make_rsrc(K + (size_t)bh * Nk * D, (uint32_t)Nk * D * 4);
    const auto rv = make_rsrc(V + (size_t)bh * Nk * D, (uint32_t)Nk * D * 4);
    const auto rl = make_rsrc(LSE + (size_t)bh * Nq, (uint32_t)Nq * 4);
    const auto rd = make_rsrc(Delta + (size_t)bh * Nq, (uint32_t)Nq * 4);

    float kq[16], vq[16];  // B operands: this lane's key row of K and of V, this wave's columns
    load_bop<4>(kq, rk, myk, D, col0, g);
    load_bop<4>(vq, rv, myk, D, col0, g);
    const bool klive = myk < Nk;

    // Causal: queries before k0 see none of these keys.
    const int qstart = CAUSAL ? k0 : 0;
    const int nsteps = qstart < Nq ? (Nq - qstart + kStep - 1) / kStep : 0;
    const int per = (nsteps + NS - 1) / NS;
    const int st0 = slice * per;
    const int st1 = min(nsteps, st0 + per);
    // with the exchange every wave runs the same number of steps (each step
    // has a barrier); past st1 they are masked
    const int st_end = CS == 2 ? st0 + per : st1;

    // [j][r] = dK (/ scale), dV of key myk, column col0 + 16g + 4r + j
    f32x4 dk[4], dv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) dk[j] = dv[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    struct Ops {
        Op<4> qr, gr;  // Q and dO by rows (first products), this wave's columns
        Op<4> qc, gc;  // Q and dO by columns (second products), this wave's columns
        f32x4 l, d;    // L and D of queries q0 + 4g .. + 3
    };
    auto load = [&](Ops &o, int q0) {
        load_rows(o.qr, rq, q0, D, col0, g, c);
        load_rows(o.gr, rdo, q0, D, col0, g, c);
        load_cols(o.qc, rq, q0, D, col0, g, c);
        load_cols(o.gc, rdo, q0, D, col0, g, c);
        o.l = __builtin_bit_cast(f32x4, load16(rl, (uint32_t)((q0 + 4 * g) * 4)));
        o.d = __builtin_bit_cast(f32x4, load16(rd, (uint32_t)((q0 + 4 * g) * 4)));
    };
    // One 16-query step on `cur`, with the next step's operands loaded into
    // `nxt` first (in-range data or zeros), so that the loads overlap this
    // step's products.
    auto step = [&](int st, int parity, const Ops &cur, Ops &nxt) {
        const int q0 = qstart + st * kStep;
        load(nxt, q0 + kStep);
        __builtin_amdgcn_sched_barrier(0);
        f32x4 s = product(cur.qr, kq);   // s[r]: S[q0 + 4g + r][myk]
        f32x4 dp = product(cur.gr, vq);  // dP, same slots
        if constexpr (CS == 2) {
            // Both waves of the pair add the same two values (addition is
            // commutative), so their P and dS agree bit for bit.  The parity
            // keeps a fast wave's next write off the buffer its partner may
            // still be reading: that write comes after the next barrier.
            s_part[parity][wave][0][lane] = s;
            s_part[parity][wave][1][lane] = dp;
            __syncthreads();
            s += s_part[parity][wave ^ 1][0][lane];
            dp += s_part[parity][wave ^ 1][1][lane];
        }
        const bool in_slice = st < st1;
        float p[4], ds[4];
        // the per-score mask only on steps that reach past Nq or Nk, cross the
        // diagonal or lie past this wave's slice (a wave-uniform test)
        if (in_slice && q0 + kStep <= Nq && k0 + kT <= Nk && !(CAUSAL && k0 + kT - 1 > q0)) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[r] = exp2f_fast(__builtin_fmaf(s[r], scale_log2, -cur.l[r] * kLog2e));
                ds[r] = p[r] * (dp[r] - cur.d[r]);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int q = q0 + 4 * g + r;
                bool live = in_slice && klive && q < Nq;
                if (CAUSAL) live = live && myk <= q;
                p[r] = live ? exp2f_fast(__builtin_fmaf(s[r], scale_log2, -cur.l[r] * kLog2e)) : 0.f;
                ds[r] = p[r] * (dp[r] - cur.d[r]);
            }
        }
        accumulate(dv, cur.gc, p);
        accumulate(dk, cur.qc, ds);
    };

    Ops ra, rb;
    load(ra, qstart + st0 * kStep);
    for (int st = st0; st < st_end; st += 2) {
        step(st, 0, ra, rb);
        step(st + 1, 1, rb, ra);
    }

#pragma unroll
    for (int r = 0; r < 4; ++r) {
        *reinterpret_cast<f32x4 *>(&s_acc[0][slice][c][col0 + 16 * g + 4 * r]) =
            f32x4{dk[0][r], dk[1][r], dk[2][r], dk[3][r]};
        *reinterpret_cast<f32x4 *>(&s_acc[1][slice][c][col0 + 16 * g + 4 * r]) =
            f32x4{dv[0][r], dv[1][r], dv[2][r], dv[3][r]};
    }
    __syncthreads();
    for (int e = threadIdx.x; e < kT * D; e += kW * 64) {
        const int row = e / D, d = e % D;
        float sk = 0.f, sv = 0.f;
#pragma unroll
        for (int w = 0; w < NS; ++w) {
            sk += s_acc[0][w][row][d];
            sv += s_acc[1][w][row][d];
        }
        if (k0 + row < Nk) {
            const size_t at = ((size_t)bh * Nk + k0 + row) * D + d;
            dK[at] = sk * scale;
            dV[at] = sv;
        }
    }
}

template <int D>
fa2_status launch_d(const BwdArgs &a, hipStream_t st) {
    const long long bh = (long long)a.B * a.H;
    const float *q = (const float *)a.q, *k = (const float *)a.k, *v = (const float *)a.v;
    const float *o = (const float *)a.o, *g = (const float *)a.dout;
    const float sl2 = a.scale * kLog2e;
    const dim3 block(kW * 64);
    fa2_status s = FA2_OK;
    if (a.Nq > 0) {
        s = launch(bwd_f32_delta_kernel<D>, dim3((a.Nq + 15) / 16, (unsigned)bh), dim3(256), st, o, g,
                   a.delta, a.Nq);
        if (s != FA2_OK) return s;
        auto kq = a.causal ? bwd_f32_dq_kernel<D, true> : bwd_f32_dq_kernel<D, false>;
        s = launch(kq, dim3((unsigned)(((a.Nq + kT - 1) / kT) * bh)), block, st, q, k, v, g, a.lse,
                   (const float *)a.delta, (float *)a.dq, a.Nq, a.Nk, a.scale, sl2);
        if (s != FA2_OK) return s;
    }
    // with no queries this still runs: it writes dK = dV = 0
    auto kk = a.causal ? bwd_f32_dkdv_kernel<D, true> : bwd_f32_dkdv_kernel<D, false>;
    return launch(kk, dim3((unsigned)(((a.Nk + kT - 1) / kT) * bh)), block, st, q, k, v, g, a.lse,
                  (const float *)a.delta, (float *)a.dk, (float *)a.dv, a.Nq, a.Nk, a.scale, sl2);
}

}  // namespace

fa2_status launch_bwd_f32(const BwdArgs &a, hipStream_t st) {
    // one-dimensional grids of 16-row tiles must fit a grid dimension
    const long long longest = a.Nq > a.Nk ? a.Nq : a.Nk;
    if ((long long)a.B * a.H * ((longest + kT - 1) / kT) > 0x7FFFFFFFLL) return FA2_ERR_UNSUPPORTED;
    if (a.D == 64) return launch_d<64>(a, st);
    if (a.D == 128) return launch_d<128>(a, st);
    return FA2_ERR_UNSUPPORTED;
}

}  // namespace fa2
