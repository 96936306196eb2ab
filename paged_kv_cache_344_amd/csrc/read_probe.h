// read_probe.h - launcher of the read-rate probe (read_probe.hip), for pa_api.cpp.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kProbeGrid = 2048;         // workgroups: eight per compute unit
constexpr int kProbeTile = 4096;         // bytes a workgroup reads per tile (16 a thread)
constexpr int kProbeWaves = 4;           // 256 threads
constexpr int kProbeTilesInFlight = 8;   // tiles a workgroup has in flight at once

// sink: kProbeGrid * kProbeWaves uint32 words, one fold per wave
hipError_t launch_read_probe(const char* src, int64_t tiles_in_src, const int32_t* tiles,
                             int64_t n_tiles, uint32_t* sink, hipStream_t stream);

}  // namespace pa
