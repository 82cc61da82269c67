// Launch sizing shared by the kernel translation units: the dynamic-LDS
// limit of a kernel and the workgroups of it that fit the device at once.
// Both are properties of (device, kernel, block size, LDS bytes) and are
// looked up once, then kept for the process, so that a call pays no runtime
// query on the host beyond the launches themselves.
#include <hip/hip_runtime.h>

#include <mutex>

#include "wtconv_internal.h"

namespace wtc {
namespace {

struct Entry {
    int dev;
    const void* fn;
    int nt;
    size_t lds;
    int resident;  // -1: only the LDS limit is recorded
};

constexpr int kEntries = 512;
std::mutex g_mutex;
Entry g_table[kEntries];
int g_count = 0;

Entry* find(int dev, const void* fn, int nt, size_t lds) {
    for (int i = 0; i < g_count; ++i) {
        Entry& e = g_table[i];
        if (e.dev == dev && e.fn == fn && e.nt == nt && e.lds == lds) return &e;
    }
    return nullptr;
}

void remember(int dev, const void* fn, int nt, size_t lds, int resident) {
    if (g_count < kEntries) g_table[g_count++] = Entry{dev, fn, nt, lds, resident};
}

}  // namespace

hipError_t prepare_lds(const void* fn, size_t lds) {
    if (lds <= 65536) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_mutex);
    // nt = 0 marks the entry of the limit itself
    if (find(dev, fn, 0, lds)) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e == hipSuccess) remember(dev, fn, 0, lds, -1);
    return e;
}

int resident_wgs(const void* fn, int nt, size_t lds) {
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 1024;
    {
        std::lock_guard<std::mutex> lock(g_mutex);
        if (const Entry* e = find(dev, fn, nt, lds)) return e->resident;
    }
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, nt, lds) != hipSuccess ||
        cus <= 0 || per <= 0)
        return 1024;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!find(dev, fn, nt, lds)) remember(dev, fn, nt, lds, cus * per);
    return cus * per;
}

}  // namespace wtc
