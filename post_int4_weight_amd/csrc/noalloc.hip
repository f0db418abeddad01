// hessian_accumulate for callers that cannot allocate device memory (code
// under HIP graph capture, tight calibration or serving loops, harnesses
// that forbid hipMalloc): the same X^T X and column sums of squares, with
// the scratch in a fixed array of device memory instead of a workspace.
//
// The array is a file-scope __device__ variable, so every GPU the library
// runs on holds its own copy at its own address for the rest of the process.
// Host code never passes the array's name to a kernel (on the host it names a
// stand-in, not device memory): the first call on a device, with that device
// current, asks the runtime for the device address and keeps it per device.
// Every call on one GPU shares that GPU's copy, so calls that overlap on one
// GPU (two streams, two threads) race; the transposed chunk and the fp64 sums
// are rewritten in full by every chunk, so no call depends on what the last
// one left there.
#include "common.hpp"

#include <mutex>

namespace ptq {
namespace {

// 64 MiB: the transposed copy of one chunk of rows and that chunk's fp64
// row-group sums (1100 rows a chunk at in = 28672, 8000 at in = 4096).
static __device__ __align__(256) unsigned char scratch[PTQ_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_scratch[MAX_DEVICES];   // device address of `scratch`, per device

int scratch_address(void** out) {
    int dev = 0;
    PTQ_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= MAX_DEVICES) {
        set_error("hessian_accumulate_noalloc: device %d outside the %d the library tracks", dev, MAX_DEVICES);
        return PTQ_EINVAL;
    }
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        PTQ_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p) {
            set_error("hessian_accumulate_noalloc: no device address for the scratch array on device %d", dev);
            return PTQ_EHIP;
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return PTQ_OK;
}

}  // namespace
}  // namespace ptq

using namespace ptq;

extern "C" int hessian_accumulate_noalloc(float* H, double* d, int64_t in, const void* X, int x_dtype,
                                          int64_t rows, int64_t ldx, void* stream) {
    const char* fn = "hessian_accumulate_noalloc";
    PTQ_TRY(check_hessian_args(fn, H, d, in, X, x_dtype, rows, ldx));
    if (x_dtype == PTQ_BF16 && xtx_bounded_chunk(in, PTQ_NOALLOC_SCRATCH_BYTES) < 64) {
        set_error("%s: in = %lld is too large: a 64-row chunk's transposed copy and sums exceed the %llu-byte "
                  "scratch (hessian_accumulate with a workspace has no such limit)",
                  fn, (long long)in, (unsigned long long)PTQ_NOALLOC_SCRATCH_BYTES);
        return PTQ_EINVAL;
    }
    if (rows == 0) return PTQ_OK;
    void* p = nullptr;
    PTQ_TRY(scratch_address(&p));
    return launch_xtx_bounded(H, d, in, X, x_dtype, rows, ldx, p, PTQ_NOALLOC_SCRATCH_BYTES, (hipStream_t)stream);
}
