// Library-wide entry points of libsdv: version and error text.
#include <stdarg.h>
#include <stdio.h>

#include "sdv_internal.h"

namespace sdv {

static thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_last_error[0] = '\0'; }

int check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SD_EDEVICE, "%s: %s", what, hipGetErrorString(e));
    return SD_OK;
}

int cu_count(const char* what, int* n) {
    static int cached = 0;
    if (cached == 0) {
        int dev = 0, c = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            c <= 0)
            return fail(SD_EDEVICE, "%s: cannot query the CU count", what);
        cached = c;
    }
    *n = cached;
    return SD_OK;
}

}  // namespace sdv

extern "C" int sd_abi_version(void) { return SD_ABI_VERSION; }

extern "C" const char* sd_last_error(void) { return sdv::g_last_error; }

extern "C" int sd_get_device_error(const int32_t* dev_error, int32_t* code, void* stream) {
    sdv::clear_error();
    if (!dev_error || !code) return sdv::fail(SD_EINVAL, "sd_get_device_error: NULL pointer");
    hipStream_t s = (hipStream_t)stream;
    int32_t word = 0;
    hipError_t e = hipMemcpyAsync(&word, dev_error, sizeof word, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess)
        return sdv::fail(SD_EDEVICE, "sd_get_device_error: %s", hipGetErrorString(e));
    *code = word;
    return SD_OK;
}
