// api.cpp -- the C ABI declared in include/fa2.h: argument checks, device
// checks and dispatch to the kernel launchers.  Nothing here allocates,
// frees or synchronises; every launch goes on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <random>

#include "fa2_internal.h"

#define FA2_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kMaxDevices = 64;
constexpr long long kMaxSliceBytes = (1LL << 31) - (1LL << 20);

// Workspace of attn_fwd_noalloc: the key-split partials of the forward live
// in this array instead of caller or library allocations.  Every device the
// library is loaded on holds its own copy, from the moment the code object is
// loaded until the process ends; all attn_fwd_noalloc calls on one device
// share it.  Host code never uses the name itself as an address (on the host
// it is only a handle): each device's address is looked up once, below.
constexpr size_t kScratchBytes = FA2_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct DeviceInfo {
    int ok = 0;
    int num_cus = 0;
    void *scratch = nullptr;  // this device's copy of `scratch` (null if the lookup failed)
};

std::once_flag g_once[kMaxDevices];
DeviceInfo g_info[kMaxDevices];

// Properties of the current device, filled once per device (thread-safe),
// with that device current: its compute units, whether it is a gfx950, and
// the device address of its scratch array.
const DeviceInfo *current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(g_once[dev], [dev] {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) return;
        g_info[dev].num_cus = p.multiProcessorCount;
        g_info[dev].ok = std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
        if (g_info[dev].ok) {
            void *ptr = nullptr;
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess)
                g_info[dev].scratch = ptr;
            else
                (void)hipGetLastError();  // leave no sticky error for the caller's next call
        }
    });
    return g_info[dev].ok ? &g_info[dev] : nullptr;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int esize(fa2_dtype dt) { return dt == FA2_F32 ? 4 : 2; }

bool valid_dtype(int dt) { return dt == FA2_F32 || dt == FA2_F16 || dt == FA2_BF16; }

}  // namespace

namespace fa2 {

// A counter with a random start, stepped by the golden-ratio increment and
// scrambled by the SplitMix64 finaliser (Steele, Lea and Flood, "Fast
// splittable pseudorandom number generators", 2014); forced odd, so never 0
// (a handshake word's resting value).
unsigned long long next_launch_tag() {
    static std::atomic<unsigned long long> state{[] {
        unsigned long long seed =
            (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count();
        seed ^= (unsigned long long)(uintptr_t)&seed;
        try {  // no exception may leave the C ABI; the clock alone is a usable start
            std::random_device rd;
            seed ^= ((unsigned long long)rd() << 32) ^ rd();
        } catch (...) {
        }
        return seed;
    }()};
    unsigned long long z = state.fetch_add(0x9E3779B97F4A7C15ull) + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (z ^ (z >> 31)) | 1ull;
}

}  // namespace fa2

namespace {

size_t fwd_workspace_bytes(int B, int H, int Nq, int Nk, int D, int causal, fa2_dtype dtype,
                           int cus) {
    if (dtype == FA2_F32) return fa2::f32_workspace_bytes(B, H, Nq, Nk, D, causal, cus);
    return fa2::mfma_workspace_bytes(B, H, Nq, Nk, D, causal, cus);
}

// use_scratch: take the device's scratch array as the workspace (shapes that
// would need more are refused).
fa2_status fwd_impl(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                    int Nq, int Nk, int D, float scale, int causal, fa2_dtype dtype,
                    void *workspace, size_t workspace_bytes, void *stream,
                    bool use_scratch = false) {
    if (B < 0 || H < 0 || Nq < 0 || Nk < 1 || D < 1) return FA2_ERR_SHAPE;
    if (!valid_dtype(dtype)) return FA2_ERR_UNSUPPORTED;
    if (causal != 0 && causal != 1) return FA2_ERR_UNSUPPORTED;
    if (!std::isfinite(scale)) return FA2_ERR_UNSUPPORTED;
    if (D != 64 && D != 128) return FA2_ERR_UNSUPPORTED;
    if (causal && Nq != Nk) return FA2_ERR_UNSUPPORTED;
    if ((long long)B * H * Nq == 0) return FA2_OK;  // nothing to compute
    if (!q || !k || !v || !o) return FA2_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
        (lse && ((uintptr_t)lse & 3u)) || (workspace && !aligned16(workspace)))
        return FA2_ERR_ALIGN;
    const long long es = esize(dtype);
    if ((long long)Nk * D * es > kMaxSliceBytes || (long long)Nq * D * es > kMaxSliceBytes)
        return FA2_ERR_UNSUPPORTED;
    if ((long long)B * H > 65535) return FA2_ERR_UNSUPPORTED;
    const DeviceInfo *dev = current_device();
    if (!dev) return FA2_ERR_DEVICE;
    if (use_scratch) {
        if (fwd_workspace_bytes(B, H, Nq, Nk, D, causal, dtype, dev->num_cus) > kScratchBytes)
            return FA2_ERR_UNSUPPORTED;
        if (!dev->scratch) return FA2_ERR_DEVICE;
        workspace = dev->scratch;
        workspace_bytes = kScratchBytes;
    }
    fa2::FwdArgs a{q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, dev->num_cus,
                   workspace, workspace ? workspace_bytes : 0};
    hipStream_t st = (hipStream_t)stream;
    if (dtype == FA2_F32) return fa2::launch_fwd_f32(a, st);
    return fa2::launch_fwd_mfma(a, dtype, st);
}

}  // namespace

FA2_API fa2_status attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                            int B, int H, int Nq, int Nk, int D, float scale, int causal,
                            fa2_dtype dtype, void *stream) {
    return fwd_impl(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, dtype, nullptr, 0, stream);
}

FA2_API fa2_status attn_fwd_ws(const void *q, const void *k, const void *v, void *o, float *lse,
                               int B, int H, int Nq, int Nk, int D, float scale, int causal,
                               fa2_dtype dtype, void *workspace, size_t workspace_bytes,
                               void *stream) {
    return fwd_impl(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, dtype, workspace,
                    workspace_bytes, stream);
}

FA2_API fa2_status attn_fwd_noalloc(const void *q, const void *k, const void *v, void *o,
                                    float *lse, int B, int H, int Nq, int Nk, int D, float scale,
                                    int causal, fa2_dtype dtype, void *stream) {
    return fwd_impl(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, dtype, nullptr, 0, stream,
                    true);
}

FA2_API size_t attn_fwd_workspace_size(int B, int H, int Nq, int Nk, int D, int causal,
                                       fa2_dtype dtype) {
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || !valid_dtype(dtype)) return 0;
    if (D != 64 && D != 128) return 0;
    if (causal && Nq != Nk) return 0;
    if ((long long)B * H > 65535) return 0;
    int cus = 256;
    if (const DeviceInfo *dev = current_device()) cus = dev->num_cus;
    return fwd_workspace_bytes(B, H, Nq, Nk, D, causal, dtype, cus);
}

FA2_API fa2_status attn_bwd(const void *q, const void *k, const void *v, const void *o,
                            const void *dout, const float *lse, void *dq, void *dk, void *dv,
                            float *delta, int B, int H, int Nq, int Nk, int D, float scale,
                            int causal, fa2_dtype dtype, void *stream) {
    if (B < 0 || H < 0 || Nq < 0 || Nk < 1 || D < 1) return FA2_ERR_SHAPE;
    if (!valid_dtype(dtype)) return FA2_ERR_UNSUPPORTED;
    if (causal != 0 && causal != 1) return FA2_ERR_UNSUPPORTED;
    if (!std::isfinite(scale)) return FA2_ERR_UNSUPPORTED;
    if (D != 64 && D != 128) return FA2_ERR_UNSUPPORTED;
    if (causal && Nq != Nk) return FA2_ERR_UNSUPPORTED;
    if ((long long)B * H == 0) return FA2_OK;
    if (!k || !v || !dk || !dv) return FA2_ERR_NULL;
    if (Nq > 0 && (!q || !o || !dout || !lse || !dq || !delta)) return FA2_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
        !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(lse) || !aligned16(delta))
        return FA2_ERR_ALIGN;
    const long long es = esize(dtype);
    if ((long long)Nk * D * es > kMaxSliceBytes || (long long)Nq * D * es > kMaxSliceBytes)
        return FA2_ERR_UNSUPPORTED;
    if ((long long)B * H > 65535) return FA2_ERR_UNSUPPORTED;
    // one workgroup per 128 query rows or per 128 keys (64 with D = 128) of
    // each (b,h): the grids hold fewer than 2^24 workgroups
    const int per_wg = D == 64 ? 128 : 64;
    if ((long long)((Nq > Nk ? Nq : Nk) + per_wg - 1) / per_wg * B * H >= (1LL << 24))
        return FA2_ERR_UNSUPPORTED;
    if (!current_device()) return FA2_ERR_DEVICE;
    fa2::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, Nq, Nk, D, scale, causal};
    if (dtype == FA2_F32) return fa2::launch_bwd_f32(a, (hipStream_t)stream);
    return fa2::launch_bwd_mfma(a, dtype, (hipStream_t)stream);
}

FA2_API fa2_status attn_decode_split(const void *q, const void *k, const void *v,
                                     float *o_part, float *m_part, float *l_part, int B, int H,
                                     int N, int D, float scale, int n_splits, fa2_dtype dtype,
                                     void *stream) {
    if (B < 0 || H < 0 || N < 1 || D < 1 || n_splits < 1) return FA2_ERR_SHAPE;
    if (!valid_dtype(dtype)) return FA2_ERR_UNSUPPORTED;
    if (!std::isfinite(scale)) return FA2_ERR_UNSUPPORTED;
    if (D != 64 && D != 128) return FA2_ERR_UNSUPPORTED;
    if ((long long)B * H == 0) return FA2_OK;
    if (!q || !k || !v || !o_part || !m_part || !l_part) return FA2_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_part) ||
        ((uintptr_t)m_part & 3u) || ((uintptr_t)l_part & 3u))
        return FA2_ERR_ALIGN;
    if ((long long)N * D * esize(dtype) > kMaxSliceBytes) return FA2_ERR_UNSUPPORTED;
    if ((long long)B * H > 65535 || n_splits > 0x7FFFFFFF / 2) return FA2_ERR_UNSUPPORTED;
    if (!current_device()) return FA2_ERR_DEVICE;
    fa2::DecodeArgs a{q, k, v, o_part, m_part, l_part, B, H, N, D, scale, n_splits};
    return fa2::launch_decode_split(a, dtype, (hipStream_t)stream);
}

FA2_API fa2_status attn_decode_combine(const float *o_part, const float *m_part,
                                       const float *l_part, void *o, int B, int H, int D,
                                       int n_splits, fa2_dtype dtype, void *stream) {
    if (B < 0 || H < 0 || D < 1 || n_splits < 1) return FA2_ERR_SHAPE;
    if (!valid_dtype(dtype)) return FA2_ERR_UNSUPPORTED;
    if (D != 64 && D != 128) return FA2_ERR_UNSUPPORTED;
    if ((long long)B * H == 0) return FA2_OK;
    if (!o_part || !m_part || !l_part || !o) return FA2_ERR_NULL;
    if (!aligned16(o_part) || ((uintptr_t)m_part & 3u) || ((uintptr_t)l_part & 3u) || !aligned16(o))
        return FA2_ERR_ALIGN;
    if ((long long)B * H > 0x7FFFFFFF) return FA2_ERR_UNSUPPORTED;
    if (!current_device()) return FA2_ERR_DEVICE;
    return fa2::launch_decode_combine(o_part, m_part, l_part, o, B, H, D, n_splits, dtype,
                                      (hipStream_t)stream);
}

FA2_API int attn_decode_default_splits(int B, int H, int N, int D) {
    (void)D;
    if (B < 1 || H < 1 || N < 1) return 1;
    int cus = 256;
    if (const DeviceInfo *dev = current_device()) cus = dev->num_cus;
    const long long bh = (long long)B * H;
    // Aim for about 8 resident workgroups per compute unit, each with at least
    // 256 keys, and round to a whole number of splits per (b,h).
    long long want = (8LL * cus + bh - 1) / bh;
    const long long max_by_len = (N + 255) / 256;
    if (want > max_by_len) want = max_by_len;
    if (want < 1) want = 1;
    return (int)want;
}

FA2_API fa2_status fa2_time_next_launch(void *start_event, void *stop_event) {
    fa2::TimingRequest &tr = fa2::timing_request();
    tr.start = (hipEvent_t)start_event;
    tr.stop = (hipEvent_t)stop_event;
    return FA2_OK;
}

FA2_API const char *fa2_status_string(fa2_status s) {
    switch (s) {
        case FA2_OK: return "ok";
        case FA2_ERR_NULL: return "null pointer";
        case FA2_ERR_SHAPE: return "invalid shape";
        case FA2_ERR_UNSUPPORTED: return "unsupported configuration";
        case FA2_ERR_ALIGN: return "pointer not 16-byte aligned";
        case FA2_ERR_LAUNCH: return "kernel launch failed";
        case FA2_ERR_DEVICE: return "no usable gfx950 device";
    }
    return "unknown status";
}
