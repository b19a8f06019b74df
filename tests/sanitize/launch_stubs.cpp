// launch_stubs.cpp -- stand-ins for the kernel launchers of pa_kernels.hip in
// the CPU-only sanitizer build of the host code (tests/test_sanitize_cpu.py).
// That build compiles pa_api.cpp with g++ and AddressSanitizer /
// UndefinedBehaviorSanitizer so that the argument checks and the plan
// builders run under them; these stand-ins launch nothing and report
// success.  They are never linked into libpa.so.
#include "pa_internal.h"

namespace pa {

hipError_t launch_write_kv(const WriteKvArgs &, hipStream_t) { return hipSuccess; }
hipError_t launch_decode_partial(const DecodeArgs &, hipStream_t) { return hipSuccess; }
hipError_t launch_decode_merge(const DecodeArgs &, hipStream_t) { return hipSuccess; }
hipError_t launch_decode_merge_planned(const DecodeArgs &, hipStream_t) { return hipSuccess; }
hipError_t launch_decode_prefix(const DecodeArgs &, hipStream_t) { return hipSuccess; }
hipError_t launch_cascade(const DecodeArgs &, hipStream_t) { return hipSuccess; }
hipError_t launch_prefill(const DecodeArgs &, hipStream_t) { return hipSuccess; }
hipError_t launch_mixed(const DecodeArgs &, hipStream_t) { return hipSuccess; }
hipError_t noalloc_scratch(hipStream_t, void **ptr) {
    *ptr = reinterpret_cast<void *>(uintptr_t{1} << 20);  // never dereferenced: nothing is launched
    return hipSuccess;
}

}  // namespace pa
