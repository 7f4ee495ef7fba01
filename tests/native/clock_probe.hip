// Measurement helper (not part of libfp8bs, not declared in fp8bs.h): stamps
// the engine-clock cycle counter and the constant-rate wall clock of every
// compute unit a grid lands on.  Two stamps around a stretch of GPU work give
// each unit's average engine clock over that stretch:
//   f = (cycles_after - cycles_before) / (wall_after - wall_before) * wall_rate.
// clock64() reads the shader cycle counter (s_memtime, counting at the XCD's
// engine clock); wall_clock64() reads the fixed-rate counter whose rate the
// runtime reports as hipDeviceAttributeWallClockRate.  The cycle counters of
// different compute units are not aligned (measured: millions of cycles apart
// within one XCD), so stamps are paired per compute unit, by the XCC_ID and
// HW_ID hardware registers, never by workgroup index.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

// s_getreg immediates (size - 1 in bits 15:11, offset in 10:6, register id in
// 5:0): XCC_ID (register 20, bits 3:0) and all 32 bits of HW_ID (register 4:
// CU in bits 11:8, SH in bit 12, SE in bits 14:13 on gfx94x/gfx950)
constexpr int kXccIdReg = (3 << 11) | (0 << 6) | 20;
constexpr int kHwIdReg = (31 << 11) | (0 << 6) | 4;

// out[3*b + 0..2] = (compute-unit key, cycle counter, wall clock) of
// workgroup b; key = XCC id * 256 + (SE, SH, CU bits of HW_ID)
__global__ __launch_bounds__(64) void clock_stamp_kernel(uint64_t* __restrict__ out) {
  if (threadIdx.x != 0) return;
  const uint32_t xcc = (uint32_t)__builtin_amdgcn_s_getreg(kXccIdReg) & 0xF;
  const uint32_t cu = ((uint32_t)__builtin_amdgcn_s_getreg(kHwIdReg) >> 8) & 0x7F;
  const uint64_t cyc = clock64();
  const uint64_t wall = wall_clock64();
  uint64_t* o = out + 3 * (uint64_t)blockIdx.x;
  o[0] = (uint64_t)(xcc * 256 + cu);
  o[1] = cyc;
  o[2] = wall;
}

}  // namespace

// Stamp `blocks` workgroups (64 threads each) into out[3 * blocks] on the
// stream.  Returns 0, or 1 if the launch failed (nothing is written then).
extern "C" int fp8bs_clock_stamp(uint64_t* out, int blocks, void* stream) {
  if (out == nullptr || blocks <= 0) return 1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(clock_stamp_kernel, dim3((unsigned)blocks), dim3(64), 0,
                     (hipStream_t)stream, out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// Rate of wall_clock64() on the current device, in kHz (0 on failure).
extern "C" int fp8bs_wall_clock_khz() {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return khz;
}
