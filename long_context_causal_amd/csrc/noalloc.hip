// cpattn_forward for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// the same launches as cpattn_forward, with the step partials in a scratch
// array that lives inside the library instead of a caller's workspace.
//
// The array is a file-scope __device__ object, so every GPU the library
// runs on holds its own copy, at its own address, from the moment the code
// object is loaded there until the process ends.  In host code the array's
// name is not a device address; its address on a device comes from
// hipGetSymbolAddress with that device current, taken once per device and
// kept.  Every call on a device uses that device's copy, and the call
// clears nothing in it: cpattn_forward_steps writes every partial it later
// merges (every row of every step's O and L) before the merge reads it.
// Calls that overlap on one device (two streams, or two host threads)
// share the array and race; the caller serialises them.
#include <hip/hip_runtime.h>

#include <mutex>

#include "cpattn.h"

namespace {

__device__ __attribute__((aligned(256))) char scratch[CPATTN_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mutex;
void *scratch_ptr[MAX_DEVICES];   // device address of each device's copy, once known

// The current device's copy of the array: looked up on the first call made
// with that device current, then reused.
int current_scratch(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return CPATTN_EHIP;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return CPATTN_EHIP;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return CPATTN_OK;
}

}  // namespace

extern "C" int cpattn_forward_noalloc(const cpattn_dims *dims, int dtype, float scale, int rank,
                                      const void *qz, const void *kz, const void *vz,
                                      int out_dtype, void *o_out, float *lse_out,
                                      void *stream) {
    // argument checks first (nothing is looked up or launched for a bad
    // call); cpattn_forward repeats them against the scratch array
    if (dims == nullptr) return CPATTN_EINVAL;
    if (dims->cp < 1 || rank < 0 || rank >= dims->cp) return CPATTN_EINVAL;
    const size_t need = cpattn_forward_workspace(dims, rank);
    if (need == 0) return CPATTN_ESHAPE;
    if (need > (size_t)CPATTN_NOALLOC_SCRATCH_BYTES) return CPATTN_ENOSPACE;
    void *ws = nullptr;
    const int st = current_scratch(&ws);
    if (st) return st;
    return cpattn_forward(dims, dtype, scale, rank, qz, kz, vz, ws,
                          (size_t)CPATTN_NOALLOC_SCRATCH_BYTES, out_dtype, o_out, lse_out,
                          stream);
}
