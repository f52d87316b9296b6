// fa2_internal.h -- launchers shared between the kernel sources and the C ABI.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include "../../include/fa2.h"

namespace fa2 {

// The calling thread's pending request from fa2_time_next_launch: the next
// launch records these events from its own dispatch, then clears them.
struct TimingRequest {
    hipEvent_t start = nullptr, stop = nullptr;
};
inline TimingRequest &timing_request() {
    static thread_local TimingRequest r;
    return r;
}

// Launch a kernel so that the runtime's verdict is returned: hipLaunchKernel,
// or hipExtLaunchKernel with the thread's pending timing events (the events
// then carry the kernel's own start and end).
template <typename... KArgs, typename... Args>
inline fa2_status launch(void (*kern)(KArgs...), dim3 grid, dim3 block, hipStream_t st,
                         Args... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
    void *ptrs[] = {(void *)&args...};
    TimingRequest &tr = timing_request();
    hipError_t e;
    if (tr.start || tr.stop) {
        const TimingRequest use = tr;
        tr = TimingRequest{};
        e = hipExtLaunchKernel((const void *)kern, grid, block, ptrs, 0, st, use.start, use.stop, 0);
    } else {
        e = hipLaunchKernel((const void *)kern, grid, block, ptrs, 0, st);
    }
    return e == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}

struct FwdArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int B, H, Nq, Nk, D;
    float scale;
    int causal;
    int num_cus;
    void *ws;         // optional device workspace (may be null)
    size_t ws_bytes;  // its size
};

// A fresh odd 64-bit value per call (never 0), for the per-launch tags of the
// in-kernel key-chunk merges; thread-safe.
unsigned long long next_launch_tag();

// float32 forward on float32 matrix cores, D = 64 or 128.
fa2_status launch_fwd_f32(const FwdArgs &a, hipStream_t st);
size_t f32_workspace_bytes(int B, int H, int Nq, int Nk, int D, int causal, int num_cus);
// f16/bf16 forward on matrix cores, D = 64 or 128.
fa2_status launch_fwd_mfma(const FwdArgs &a, fa2_dtype dt, hipStream_t st);
size_t mfma_workspace_bytes(int B, int H, int Nq, int Nk, int D, int causal, int num_cus);

struct BwdArgs {
    const void *q, *k, *v, *o, *dout;
    const float *lse;
    void *dq, *dk, *dv;
    float *delta;
    int B, H, Nq, Nk, D;
    float scale;
    int causal;
};

// f16/bf16 backward on matrix cores, D = 64 or 128.
fa2_status launch_bwd_mfma(const BwdArgs &a, fa2_dtype dt, hipStream_t st);
// float32 backward on float32 matrix cores, D = 64 or 128.
fa2_status launch_bwd_f32(const BwdArgs &a, hipStream_t st);

struct DecodeArgs {
    const void *q, *k, *v;
    float *o_part, *m_part, *l_part;
    int B, H, N, D;
    float scale;
    int n_splits;
};

fa2_status launch_decode_split(const DecodeArgs &a, fa2_dtype dt, hipStream_t st);
// Merge per-row partials [rows][n_splits][D] (natural-log m) into o [rows][D]
// of dtype dt and, if lse is not null, lse [rows].  O is divided by the merged
// l_part; the LSE uses the merged l2_part when it is given, else l_part.
fa2_status launch_combine_rows(const float *o_part, const float *m_part, const float *l_part,
                               void *o, float *lse, size_t rows, int D, int n_splits, fa2_dtype dt,
                               hipStream_t st, const float *l2_part = nullptr);
fa2_status launch_decode_combine(const float *o_part, const float *m_part, const float *l_part,
                                 void *o, int B, int H, int D, int n_splits, fa2_dtype dt,
                                 hipStream_t st);

}  // namespace fa2
