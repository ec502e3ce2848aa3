// attn_device.hip -- device queries of the C ABI that launch nothing.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/attn.h"

// Dense fp16/bf16 matrix-core peak: each of a compute unit's four SIMDs retires one
// v_mfma_f32_32x32x16_{f16,bf16} (2*32*32*16 = 32768 flop) per 8 passes of 4 clocks
// (32 clocks), i.e. 1024 flop per clock per SIMD and 4096 per compute unit.
extern "C" int attn_device_peak(double* tflops, int32_t* compute_units, int32_t* clock_khz) {
  int dev = 0, cus = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeClockRate, dev) != hipSuccess)
    return ATTN_E_LAUNCH;
  if (compute_units) *compute_units = cus;
  if (clock_khz) *clock_khz = khz;
  if (tflops) *tflops = static_cast<double>(cus) * khz * 1e3 * 4096.0 / 1e12;
  return ATTN_OK;
}
