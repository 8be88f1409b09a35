// Host-only stand-ins for the device side of libkvdecode (the kernel launchers, the static
// workspace lookup and the two HIP device queries the C-ABI layer makes), so that the C-ABI
// layer can be built and exercised under AddressSanitizer and UndefinedBehaviorSanitizer on a
// machine without a GPU.  Each launcher records what it was given; nothing is launched.
#pragma once

#include <stdint.h>

#include "kvd_internal.h"

namespace stub {

enum Kind { kNone, kPartitions, kReduce, kGather, kOperands, kAppend, kProbe };

struct Record {
    int calls[7];
    int fmt;
    bool wide;
    dim3 grid;
    int blocks, loads_in_flight;
    kvd::LaunchParams lp;
    kvd::GatherParams gp;
    kvd::OperandParams op;
    kvd::AppendParams ap;
    kvd::ProbeParams pp;
};

extern Record rec;
extern int device_cus;          // what hipDeviceGetAttribute reports (<= 0: the query fails)
extern void* noalloc_address;   // what noalloc_workspace hands out

void reset();

}  // namespace stub
