// Knobs of the stand-in device side (stub_device.cpp).
#pragma once
namespace stub {
extern int launch_error;   // returned by every launcher
extern int pending_error;  // an error "left pending" by the caller's earlier device calls
extern int device_error;   // returned by the current-device query
extern int launches;       // launchers called so far
extern int taken;          // pending-error queries so far
extern const char* arch;   // architecture name the device reports
extern void* last_ws;      // workspace the last grouped-GEMM launch received
extern int copies;         // strided copies queued
}  // namespace stub
