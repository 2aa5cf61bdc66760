// The chunked forward without any allocation by the caller or the library: the per-chunk
// intermediates (the packed schedule and the Stage 2 records) go to a fixed scratch array
// in device memory that the code object itself holds, one copy per GPU, for callers that
// cannot allocate (code under HIP graph capture, serving loops, harnesses that forbid it).
//
// `scratch` is a device symbol: in host code its name is only a stand-in, so the host
// never passes it to a kernel. Its device address is looked up once per GPU, with that
// GPU current, on the first call there, and that address is what the kernels receive.
#include <mutex>

#include "kda_internal.h"

namespace {

constexpr size_t SCRATCH_BYTES = (size_t)KDA_NOALLOC_SCRATCH_MB << 20;
constexpr int MAX_DEVICES = 64;

static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

std::mutex g_scratch_lock;
void* g_scratch_ptr[MAX_DEVICES] = {};

// The scratch array's address on the current device (looked up on first use there).
hipError_t scratch_address(void** out) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> guard(g_scratch_lock);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) & 255) != 0) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

size_t kda_noalloc_scratch_bytes(void) { return SCRATCH_BYTES; }

int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g,
                          const void* beta, const float* initial_state,
                          const int32_t* cu_seqlens, int N, void* o, float* final_state, int B,
                          int T, int H, int HV, int K, int V, int qkv_dtype, int beta_dtype,
                          float scale, int chunk_size, int32_t* dev_status,
                          hipStream_t stream) {
    // the size check comes first and touches no GPU state; invalid sizes (need == 0) are
    // left to the forward's own validation below
    const size_t need = kda_chunk_fwd_workspace_bytes(B, T, H, HV, K, V, N, cu_seqlens != nullptr,
                                                      qkv_dtype);
    if (need > SCRATCH_BYTES)
        return kda::set_error(KDA_ERR_WORKSPACE,
                              "this problem needs %zu bytes of intermediates; the allocation-free "
                              "entry point holds %zu bytes per GPU (use kda_chunk_fwd with a "
                              "caller workspace)",
                              need, SCRATCH_BYTES);
    void* ws = nullptr;
    if (need > 0) {
        // argument errors first, without touching the GPU: with no workspace the forward
        // validates everything and stops at the missing workspace, having enqueued nothing
        const int rc = kda_chunk_fwd(q, k, v, g, beta, initial_state, cu_seqlens, N, o, final_state,
                                     B, T, H, HV, K, V, qkv_dtype, beta_dtype, scale, chunk_size,
                                     nullptr, 0, dev_status, stream);
        if (rc != KDA_ERR_WORKSPACE) return rc;
        const hipError_t err = scratch_address(&ws);
        if (err != hipSuccess)
            return kda::set_error(KDA_ERR_HIP, "scratch array address: %s", hipGetErrorString(err));
    }
    // every word of the scratch array a call reads is written earlier in that call (the
    // schedule by the scheduler kernel, each record by Stage 1+2), so nothing is cleared
    return kda_chunk_fwd(q, k, v, g, beta, initial_state, cu_seqlens, N, o, final_state, B, T, H,
                         HV, K, V, qkv_dtype, beta_dtype, scale, chunk_size, ws, SCRATCH_BYTES,
                         dev_status, stream);
}

}  // extern "C"
