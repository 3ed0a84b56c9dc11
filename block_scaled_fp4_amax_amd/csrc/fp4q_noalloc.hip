// fp4q_noalloc.hip -- fp4_qdq_noalloc: fp4_qdq for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  The scratch that fp4_qdq takes from the
// caller's workspace -- the tensorwise mode's partial maxima and its global
// scale -- lives here in a file-scope device array instead.
//
// The array's name is only a host-side stand-in on the host: its device
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and that address, never the name, is what the kernels get.
// Every call on a device shares that device's array, which keeps the last
// call's contents; nothing in it needs to start at zero (each call writes the
// partial maxima it later reads).  Calls that overlap on one device race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/fp4q.h"

namespace {

// Bytes of device scratch: at least what fp4q_workspace_bytes() reports for
// any fp4_qdq configuration (the tensorwise partial maxima: 513 floats).
constexpr size_t kScratchBytes = 4096;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

struct ScratchTable {
    std::mutex mu;
    void* ptr[kMaxDevices] = {};
};

ScratchTable& table()
{
    static ScratchTable t;
    return t;
}

// Device address of `scratch` on the current device (looked up on first use
// per device), or NULL with *err set.
void* scratch_ptr(int* err)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *err = FP4Q_ERR_HIP;
        return nullptr;
    }
    ScratchTable& t = table();
    std::lock_guard<std::mutex> lock(t.mu);
    if (t.ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            *err = FP4Q_ERR_HIP;
            return nullptr;
        }
        t.ptr[dev] = p;
    }
    return t.ptr[dev];
}

}  // namespace

extern "C" int fp4_qdq_noalloc(const fp4q_cfg* cfg, const void* x, int64_t rows, int64_t cols, int64_t ld_x, void* y,
                               uint8_t* codes, uint8_t* scales, float* outer, float* residual, void* stream)
{
    const size_t need = fp4q_workspace_bytes(cfg, rows, cols);
    if (need > kScratchBytes) return FP4Q_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        int err = FP4Q_OK;
        ws = scratch_ptr(&err);
        if (!ws) return err;
    }
    return fp4_qdq(cfg, x, rows, cols, ld_x, y, codes, scales, outer, residual, ws, need, stream);
}
