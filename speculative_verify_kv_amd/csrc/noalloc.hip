// swattn_verify_noalloc: swattn_verify for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  The split plans' workspace (arrival counters, partial outputs and
// their log2-sum-exps) lives in a file-scope device array instead of a caller's
// buffer; nothing is allocated or freed, by this call or by any routine it calls.
//
// The array is one per GPU and lives until the process ends.  Its device address is
// taken once per device, with that device current, by hipGetSymbolAddress: in host
// code the array's name is only a host-side stand-in, never a device address.  Every
// call on a GPU shares that GPU's array and finds what the last call left: the
// arrival counters, the only part that must start at zero, are zeroed by a fill
// kernel (not a memset, so that a graph may capture it) enqueued on the first call on
// each device that uses them, and every call leaves them zero.  Calls that overlap in
// time on one GPU (other streams, other threads) race on the array.

#include <hip/hip_runtime.h>

#include <mutex>

#include "swattn.h"
#include "swattn_internal.h"

namespace swattn {
namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[SWATTN_STATIC_SCRATCH_BYTES];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];    // device address of `scratch` on each device
bool g_scratch_zeroed[kMaxDevices];  // its arrival counters' zeroing has been enqueued

int current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
    return dev;
}

// Set-up of device `dev` (current): the device address of its `scratch`, taken once.
swattn_status_t scratch_address(int dev, void** ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SWATTN_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return SWATTN_OK;
}

// Zeroes the arrival counters on `stream` the first time a call on `dev` uses them.
swattn_status_t zero_counters_once(int dev, void* ptr, void* stream) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_zeroed[dev]) return SWATTN_OK;
    if (launch_zero_words(reinterpret_cast<int32_t*>(ptr), SWATTN_WORKSPACE_COUNTER_BYTES / 4, stream) != 0)
        return SWATTN_ERR_HIP;
    g_scratch_zeroed[dev] = true;
    return SWATTN_OK;
}

}  // namespace
}  // namespace swattn

extern "C" swattn_status_t swattn_verify_noalloc(const swattn_desc_t* d, const void* q, const void* k_cache,
                                                 const void* v_cache, const int32_t* block_table,
                                                 const int32_t* ctx_len, int32_t n_q, int32_t window, float scale,
                                                 void* out, void* stream) {
    using namespace swattn;
    swattn_plan_t plan;
    swattn_status_t st = make_plan(d, n_q, window, SWATTN_MAX_NQ, &plan);
    if (st != SWATTN_OK) return st;
    if (plan.workspace_bytes > SWATTN_STATIC_SCRATCH_BYTES) return SWATTN_ERR_SCRATCH;
    void* ws = nullptr;
    int dev = -1;
    if (plan.workspace_bytes > 0) {
        dev = current_device();
        if (dev < 0) return SWATTN_ERR_HIP;
        st = scratch_address(dev, &ws);
        if (st != SWATTN_OK) return st;
    }
    // every check first: nothing is enqueued when one fails
    AttendCall call;
    st = prepare_attend(d, q, k_cache, v_cache, block_table, ctx_len, n_q, window, scale, out, ws,
                        ws ? (size_t)SWATTN_STATIC_SCRATCH_BYTES : 0, SWATTN_MAX_NQ, &call);
    if (st != SWATTN_OK) return st;
    if (ws) {
        st = zero_counters_once(dev, ws, stream);
        if (st != SWATTN_OK) return st;
    }
    return launch_attend(call, stream);
}
