// Internal interface of the HBM bandwidth probe (kernels in hbm_probe.hip, front end in
// hyb_api.cpp, declarations and argument rules in include/hyb_probe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hyb {

enum ProbeVariant : int32_t {
  kProbeRead = 0,
  kProbeReadDyn = 1,
  kProbeReadLds = 2,
  kProbeReadPages = 3,
  kProbeCopy = 4,
};

struct ProbeArgs {
  const uint8_t* src;
  uint8_t* dst;
  uint64_t bytes;
  uint32_t* counter;      // read_dyn: chunks taken so far (zero at launch)
  const int32_t* pages;   // read_pages: page list
  int32_t n_pages;
  int64_t chunk_bytes;    // read_dyn: bytes per grab; read_pages: page size
  uint64_t* trace;        // optional [n_wg][4]: XCC id, start tick, end tick, bytes
  uint32_t* sink;         // optional [n_wg * 256]
};

uint64_t probe_granule(int variant, int unroll);
hipError_t launch_probe(int variant, int unroll, int n_wg, const ProbeArgs& a, hipStream_t s);

}  // namespace hyb
