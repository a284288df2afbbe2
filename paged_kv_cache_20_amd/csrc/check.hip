// check.hip -- checked mode on the device: validates the lengths and the
// block-table entries a call will read, writing one error word the caller
// reads after the call ("kern manifest v7" schema, $defs.Domain: the runtime
// rejects out-of-domain inputs; $defs.Fill "error": a one-word error flag read
// after every call).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace pa {
namespace {

constexpr int64_t kNoError = INT64_MAX;

__global__ void check_init(int64_t* err) { *err = kNoError; }

// One thread per (sequence, table entry); entry -1 stands for the length
// check.  Key of a failure: s * (max_pages + 1) + entry + 1, so the smallest
// key names the first failing sequence and, in it, the length before the
// first bad entry.
__global__ __launch_bounds__(256) void check_kernel(CheckArgs a)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t per = (int64_t)a.max_pages + 1;
    if (i >= (int64_t)a.n_seq * per)
        return;
    const int s = (int)(i / per);
    const int e = (int)(i - (int64_t)s * per) - 1;
    const int C = a.ctx_lens[s];
    const bool len_ok = C >= a.rows && (int64_t)C <= (int64_t)a.max_pages * a.page_size;
    bool bad;
    if (e < 0) {
        bad = !len_ok;
    } else {
        // first key the call's first row attends (window and floor)
        int first = a.kv_floor ? a.kv_floor[s] : 0;
        if (a.window > 0 && C - a.rows - a.window + 1 > first)
            first = C - a.rows - a.window + 1;
        // pages holding a key the call's rows attend (all of them when the
        // length is bad: nothing would be read)
        const bool read = len_ok && e < (C + a.page_size - 1) / a.page_size &&
                          (e + 1) * a.page_size > first;
        const int p = read ? a.block_table[(int64_t)s * a.max_pages + e] : 0;
        bad = read && (p < 0 || (int64_t)p >= a.n_pages);
    }
    if (bad)
        atomicMin((unsigned long long*)a.err, (unsigned long long)(i));
}

__global__ void check_finish(int64_t* err)
{
    if (*err == kNoError)
        *err = -1;
}

}  // namespace

hipError_t launch_check(const CheckArgs& a, hipStream_t stream)
{
    hipLaunchKernelGGL(check_init, dim3(1), dim3(1), 0, stream, a.err);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t n = (int64_t)a.n_seq * ((int64_t)a.max_pages + 1);
    hipLaunchKernelGGL(check_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(check_finish, dim3(1), dim3(1), 0, stream, a.err);
    return hipGetLastError();
}

}  // namespace pa
