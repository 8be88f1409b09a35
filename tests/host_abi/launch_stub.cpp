// Host-only stand-ins for the device side of libkvdecode; see launch_stub.h.
#include "launch_stub.h"

namespace stub {

Record rec;
int device_cus = 256;
alignas(256) static unsigned char noalloc_area[256];
void* noalloc_address = noalloc_area;

void reset() { rec = Record{}; }

}  // namespace stub

extern "C" hipError_t hipGetDevice(int* device) {
    *device = 0;
    return hipSuccess;
}

extern "C" hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int device) {
    if (attr != hipDeviceAttributeMultiprocessorCount || device != 0 || stub::device_cus <= 0)
        return hipErrorInvalidValue;
    *value = stub::device_cus;
    return hipSuccess;
}

namespace kvd {

hipError_t launch_partitions(int fmt, bool wide, const LaunchParams& p, dim3 grid, hipStream_t) {
    stub::rec.calls[stub::kPartitions]++;
    stub::rec.fmt = fmt;
    stub::rec.wide = wide;
    stub::rec.grid = grid;
    stub::rec.lp = p;
    return hipSuccess;
}

hipError_t launch_reduce(int fmt, const LaunchParams& p, hipStream_t) {
    stub::rec.calls[stub::kReduce]++;
    stub::rec.fmt = fmt;
    stub::rec.lp = p;
    return hipSuccess;
}

hipError_t launch_gather(const GatherParams& p, hipStream_t) {
    stub::rec.calls[stub::kGather]++;
    stub::rec.gp = p;
    return hipSuccess;
}

hipError_t launch_operands(int fmt, const OperandParams& p, hipStream_t) {
    stub::rec.calls[stub::kOperands]++;
    stub::rec.fmt = fmt;
    stub::rec.op = p;
    return hipSuccess;
}

hipError_t launch_append(const AppendParams& p, hipStream_t) {
    stub::rec.calls[stub::kAppend]++;
    stub::rec.ap = p;
    return hipSuccess;
}

hipError_t launch_read_probe(const ProbeParams& p, int blocks, int loads_in_flight, hipStream_t) {
    stub::rec.calls[stub::kProbe]++;
    stub::rec.pp = p;
    stub::rec.blocks = blocks;
    stub::rec.loads_in_flight = loads_in_flight;
    return hipSuccess;
}

hipError_t noalloc_workspace(void** ptr) {
    *ptr = stub::noalloc_address;
    return hipSuccess;
}

}  // namespace kvd
