// dispatch_probe.hip -- test-only probe of how a launch's workgroups reach
// the compute units, the premise behind the row-group launch plan (which XCD
// runs workgroup i; how each XCD deals its workgroups to its shader engines).
//
// Every workgroup is 1024 lanes with 96 KB of LDS, so one compute unit holds
// one at a time, as it holds one row-group workgroup.  Thread 0 reads the
// XCC_ID and HW_ID hardware registers, holds the workgroup for a number of
// ticks of the 100 MHz realtime counter (long_ticks on shader engine 0,
// short_ticks elsewhere: a bounded wait that no other workgroup affects) and
// stores one record.  Nothing here waits for another workgroup.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

struct Record {
  uint64_t xcc;   // XCC_ID register
  uint64_t hwid;  // HW_ID register: CU_ID [11:8], SH_ID [12], SE_ID [14:13]
  uint64_t t0;    // realtime counter at the start of the hold
  uint64_t t1;    // realtime counter at its end
};

__global__ __launch_bounds__(1024) void dispatch_probe(Record* out, int32_t n, uint32_t long_ticks,
                                                       uint32_t short_ticks) {
  __shared__ uint32_t lds[98304 / 4];
  lds[threadIdx.x] = threadIdx.x;
  __syncthreads();
  if (threadIdx.x != 0 || blockIdx.x >= static_cast<uint32_t>(n)) return;
  uint32_t xcc, hw;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
  const uint32_t engine = (hw >> 13) & 3u;
  const uint32_t hold = engine == 0 ? long_ticks : short_ticks;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  uint64_t t1 = t0;
  while (t1 - t0 < hold) {
    __builtin_amdgcn_s_sleep(2);
    t1 = __builtin_amdgcn_s_memrealtime();
  }
  Record r;
  r.xcc = xcc;
  r.hwid = hw;
  r.t0 = t0;
  r.t1 = t1 + (lds[1] - 1u);  // adds 0 (lds[1] is 1) and keeps the LDS allocation
  out[blockIdx.x] = r;
}

}  // namespace

// Launches n workgroups on `stream`; records[n] (device memory, 32 bytes
// each) receives one record per workgroup.  Returns the HIP error code of
// the launch (0 on success); the caller synchronises.
extern "C" int ets_test_dispatch_probe(void* records, int32_t n, uint32_t long_ticks, uint32_t short_ticks,
                                       void* stream) {
  if (records == nullptr || n <= 0) return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(dispatch_probe, dim3(static_cast<uint32_t>(n)), dim3(1024), 0,
                     static_cast<hipStream_t>(stream), static_cast<Record*>(records), n, long_ticks,
                     short_ticks);
  return static_cast<int>(hipGetLastError());
}
