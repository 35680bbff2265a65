// LDS access-pattern calibration for the bank-conflict counters.
//
// rocprofv3's SQ_LDS_BANK_CONFLICT counts cycles an LDS instruction spends
// beyond its first, so 128-bit accesses register "conflicts" even when every
// lane hits its own banks.  This program runs one kernel per lane-address
// pattern of libsfa's LDS rows (plus a contiguous reference and an unpadded
// control), each 2000 dependent ds_read_b128 or ds_write_b128 per lane, so a
// counter run shows which patterns cost more than the contiguous one:
//   contiguous      lane * 16 B
//   q1_rows         8 lanes per 272-byte row, 32 B apart (fp32 rows of
//                   D = 64 plus a 16-byte pad; query pass with one head per
//                   KV head, and every fp32 staging write)
//   q4_rows         16 lanes per 272-byte row, 16 B apart (query pass, G >= 4)
//   h16_rows        8 lanes per 144-byte row (f16 rows of D = 64 plus pad:
//                   the forward's staged rows)
//   key_rows        one 144-byte row per lane (the bf16 key pass's ring)
//   unpadded_rows   8 lanes per 256-byte row, 32 B apart (the q1 pattern
//                   without the pad: the control that does conflict)
// Prints the event time of each kernel.  Built by build.py next to libsfa.so.
#include <hip/hip_runtime.h>

#include <cstdio>

namespace {

enum Pattern { kContiguous, kQ1Rows, kQ4Rows, kH16Rows, kKeyRows, kUnpaddedRows, kNumPatterns };
const char* const kNames[kNumPatterns] = {"contiguous", "q1_rows", "q4_rows", "h16_rows", "key_rows",
                                          "unpadded_rows"};

// Byte address of a lane's 16-byte access; at most 63 * 144 + 16 < 9216.
template <int P>
__device__ __forceinline__ int lane_addr(int lane) {
  if constexpr (P == kContiguous) return lane * 16;
  if constexpr (P == kQ1Rows) return (lane / 8) * 272 + (lane % 8) * 32;
  if constexpr (P == kQ4Rows) return (lane / 16) * 272 + (lane % 16) * 16;
  if constexpr (P == kH16Rows) return (lane / 8) * 144 + (lane % 8) * 16;
  if constexpr (P == kKeyRows) return lane * 144;
  return (lane / 8) * 256 + (lane % 8) * 32;
}

constexpr int kFloats = 8192;       // 32 KiB of LDS per workgroup

template <int P, bool WRITE>
__global__ __launch_bounds__(256) void lds_pattern_kernel(float* out, int iters) {
  __shared__ __align__(16) float lds[kFloats];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int t = threadIdx.x; t < kFloats; t += 256) lds[t] = float(t);
  __syncthreads();
  // wave w uses bytes [w * 7168, w * 7168 + 9216): the last ends at 30720
  int a = (lane_addr<P>(lane) + wave * 7168) / 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int it = 0; it < iters; ++it) {
    asm volatile("" : "+v"(a));  // an opaque address: one access per iteration
    if constexpr (WRITE) {
      *reinterpret_cast<float4*>(lds + a) = make_float4(float(it), acc.y, acc.z, acc.w);
    } else {
      const float4 v = *reinterpret_cast<const float4*>(lds + a);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): each access completes before the next
  }
  __syncthreads();
  out[blockIdx.x * 256 + threadIdx.x] = acc.x + acc.y + acc.z + acc.w + lds[a];
}

constexpr int kBlocks = 1024;

template <int P, bool W>
int run(float* out) {
  hipLaunchKernelGGL((lds_pattern_kernel<P, W>), dim3(kBlocks), dim3(256), 0, 0, out, 2000);
  if (hipDeviceSynchronize() != hipSuccess) return 1;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
  (void)hipEventRecord(e0, 0);
  hipLaunchKernelGGL((lds_pattern_kernel<P, W>), dim3(kBlocks), dim3(256), 0, 0, out, 2000);
  (void)hipEventRecord(e1, 0);
  if (hipEventSynchronize(e1) != hipSuccess) return 1;
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, e0, e1);
  std::printf("%-14s %-5s %8.1f us\n", kNames[P], W ? "write" : "read", ms * 1e3f);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return 0;
}

template <int P>
int run_both(float* out) {
  return run<P, false>(out) | run<P, true>(out);
}

}  // namespace

int main() {
  float* out = nullptr;
  if (hipMalloc(&out, size_t(kBlocks) * 256 * sizeof(float)) != hipSuccess) return 1;
  int rc = 0;
  rc |= run_both<kContiguous>(out);
  rc |= run_both<kQ1Rows>(out);
  rc |= run_both<kQ4Rows>(out);
  rc |= run_both<kH16Rows>(out);
  rc |= run_both<kKeyRows>(out);
  rc |= run_both<kUnpaddedRows>(out);
  (void)hipFree(out);
  return rc;
}
