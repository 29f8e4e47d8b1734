// Fault injection and call records of the stub launchers (stubs.cpp).
#pragma once
#include <string>
#include <vector>

#include <hip/hip_runtime.h>

namespace stub {
extern std::vector<std::string> calls;  // launcher names, in call order
extern int fail_at;                     // index of the launcher call that returns fail_code (-1: none)
extern hipError_t fail_code;
extern int syncs;                       // hipStreamSynchronize calls
extern int sync_fail_at;                // index of the synchronization that returns sync_code (-1: none)
extern hipError_t sync_code;
extern hipError_t event_code;           // returned by hipEventRecord
extern hipError_t device_code;          // returned by hipGetDevice
extern hipError_t symbol_code;          // returned by hipGetSymbolAddress
extern int device;                      // the device hipGetDevice reports
extern int symbol_lookups;              // hipGetSymbolAddress calls
extern void* workspace_seen;            // a workspace slice the last linear (or attention) launch received
void reset();
}  // namespace stub
