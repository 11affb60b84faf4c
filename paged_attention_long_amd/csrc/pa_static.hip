// paged_attn_forward_noalloc: the forward for callers that cannot allocate
// device memory (code under graph capture, serving loops that forbid it).
//
// The split partials, merge descriptors and counters live in `scratch`, a
// fixed device array of PA_NOALLOC_SCRATCH_BYTES that every GPU the library
// runs on holds until the process ends.  Its device address is taken once
// per device (hipGetSymbolAddress, with that device current) and kept; host
// code never passes the array's own name to a kernel, since on the host it
// only stands in for the symbol.  Each call lays the workspace out for the
// kernels it launches, rejects a configuration that needs more than the
// array holds, and zeroes the counters the kernels expect at zero with a
// small kernel on the caller's stream.  Calls that overlap on one GPU share
// the array and race.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "paged_attn.h"
#include "pa_host.h"
#include "pa_kernels.h"

namespace pa {
namespace {

static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device (null: not yet taken)
int g_cu_count[kMaxDevices];

__global__ void zero_words_kernel(int* p, size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0;
}

// The device address of `scratch` and the CU count of the current device,
// set up on the first call on that device.
int scratch_for_device(int dev, void** ptr, int* cu) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(nullptr, PA_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                        hipGetErrorString(e));
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
        g_cu_count[dev] = n;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    *cu = g_cu_count[dev];
    return PA_OK;
}

}  // namespace

hipError_t launch_zero_words(int* p, size_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const int threads = 256;
    const size_t blocks = (n + threads - 1) / threads;
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(threads), 0, stream,
                       p, n);
    return hipGetLastError();
}

}  // namespace pa

using namespace pa;

extern "C" int paged_attn_forward_noalloc(const pa_config_t* cfg, const void* q, int64_t num_tokens,
                                          const void* k_cache, const void* v_cache, const pa_cache_layout_t* layout,
                                          const int32_t* block_table, int32_t num_seqs, int32_t block_table_stride,
                                          const int32_t* seq_lens, const int32_t* q_lens, int32_t window,
                                          float scale, const float* kv_scale, float* out, float* lse, void* stream) {
    char why[256];
    int rc = validate_config(cfg, why, sizeof why);
    if (rc != PA_OK) return fail(nullptr, rc, "%s", why);
    if (cfg->device >= kMaxDevices) return fail(nullptr, PA_ERR_UNSUPPORTED, "device %d >= %d", cfg->device, kMaxDevices);
    if (cfg->flags & PA_DEBUG_CHECKS)
        return fail(nullptr, PA_ERR_UNSUPPORTED, "PA_DEBUG_CHECKS needs a handle (its error word belongs to it)");
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= cfg->device)
        return fail(nullptr, PA_ERR_INVALID_ARGUMENT, "device %d not present (%d devices)", cfg->device, ndev);
    DeviceGuard guard(cfg->device);
    if (!guard.ok) return fail(nullptr, PA_ERR_HIP, "hipSetDevice(%d) failed", cfg->device);
    void* base = nullptr;
    int cu = 0;
    rc = scratch_for_device(cfg->device, &base, &cu);
    if (rc != PA_OK) return rc;

    // A handle on the stack: the configuration's sizing, default tuning, the
    // workspace bound into the fixed array.
    pa_handle h;
    size_handle(&h, cfg, cu);
    const ForwardCall f{q,        num_tokens, k_cache, v_cache,  layout, block_table, num_seqs, block_table_stride,
                        seq_lens, q_lens,     window,  scale,    kv_scale, out,       lse,      static_cast<hipStream_t>(stream)};
    rc = check_forward(&h, f);
    if (rc != PA_OK) return fail(nullptr, rc, "%s", h.err);
    const LaunchPlan lp = plan_launches(&h, f);
    const WsLayout L = layout_workspace(&h, lp.run_valu, lp.run_mfma);
    if (L.total > (size_t)PA_NOALLOC_SCRATCH_BYTES)
        return fail(nullptr, PA_ERR_UNSUPPORTED,
                    "this configuration needs %zu bytes of workspace; the no-allocation entry point holds %zu "
                    "(use a handle from paged_attn_create)",
                    L.total, (size_t)PA_NOALLOC_SCRATCH_BYTES);
    bind_workspace(&h, base, L);
    const hipError_t e = launch_zero_words(reinterpret_cast<int*>(static_cast<char*>(base) + L.zero_begin),
                                           (L.zero_end - L.zero_begin) / sizeof(int), f.stream);
    if (e != hipSuccess) return fail(nullptr, PA_ERR_HIP, "scratch clear failed: %s", hipGetErrorString(e));
    rc = enqueue_forward(&h, f, lp);
    if (rc != PA_OK) return fail(nullptr, rc, "%s", h.err);
    return PA_OK;
}
