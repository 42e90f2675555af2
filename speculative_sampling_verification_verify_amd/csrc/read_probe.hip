// Streaming-read ceiling of this GPU on a given pair of buffers: every 16-byte
// unit of both buffers is read once with a non-temporal load and folded into
// a per-thread checksum.  A thread writes only when its checksum equals a
// value that the host passes and no data produces in practice, so the loads
// stay and the kernel's HBM traffic is the buffers' bytes.  It computes
// nothing of the verify step: it measures what a plain read of the verify's
// logit buffers reaches, the practical ceiling for the kernels that stream
// them.
//
// Each workgroup (256 threads) reads one contiguous chunk of the two buffers
// taken as one sequence of units; UNR units per thread are in flight per step.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int PROBE_NT = 256;

template <int UNR>
__global__ __launch_bounds__(PROBE_NT) void read_probe_kernel(const u32x4* a, long long na, const u32x4* b,
                                                              long long nb, long long chunk, uint32_t never,
                                                              uint32_t* out) {
  const long long n = na + nb;
  const long long begin = (long long)blockIdx.x * chunk;
  const long long end = begin + chunk < n ? begin + chunk : n;
  u32x4 acc = {0u, 0u, 0u, 0u};
  long long i = begin + threadIdx.x;
  // Full steps: every load of the step is in range.
  for (; i + (long long)(UNR - 1) * PROBE_NT < end; i += (long long)UNR * PROBE_NT) {
    u32x4 v[UNR];
#pragma unroll
    for (int r = 0; r < UNR; ++r) {
      const long long j = i + (long long)r * PROBE_NT;
      v[r] = __builtin_nontemporal_load(j < na ? a + j : b + (j - na));
    }
#pragma unroll
    for (int r = 0; r < UNR; ++r) acc ^= v[r];
  }
  for (; i < end; i += PROBE_NT) acc ^= __builtin_nontemporal_load(i < na ? a + i : b + (i - na));
  const uint32_t h = acc.x ^ (acc.y * 3u) ^ (acc.z * 5u) ^ (acc.w * 7u);
  if (h == never) out[blockIdx.x] = h;
}

}  // namespace

// Reads a_bytes of `a` and b_bytes of `b` (device pointers, 16-byte aligned,
// sizes multiples of 16) in `grid` workgroups with `unroll` (4, 8 or 16) units
// per thread in flight, on `stream`.  `out` ([grid] uint32) is written only in
// the case described above.  Returns 0, -1 for bad arguments, or -4 when the
// launch fails.
extern "C" int sv_read_probe(const void* a, size_t a_bytes, const void* b, size_t b_bytes, uint32_t* out, int grid,
                             int unroll, uint32_t never, void* stream) {
  if (!a || !out || grid < 1 || (a_bytes % 16) || (b_bytes % 16) || ((uintptr_t)a % 16) ||
      (b_bytes && (!b || ((uintptr_t)b % 16))))
    return -1;
  const long long na = (long long)(a_bytes / 16), nb = (long long)(b_bytes / 16);
  const long long per = (na + nb + grid - 1) / grid;
  const long long chunk = (per + PROBE_NT - 1) / PROBE_NT * PROBE_NT;
  const u32x4* pa = reinterpret_cast<const u32x4*>(a);
  const u32x4* pb = reinterpret_cast<const u32x4*>(b ? b : a);
  hipStream_t st = (hipStream_t)stream;
  switch (unroll) {
    case 4: hipLaunchKernelGGL(read_probe_kernel<4>, dim3(grid), dim3(PROBE_NT), 0, st, pa, na, pb, nb, chunk, never, out); break;
    case 8: hipLaunchKernelGGL(read_probe_kernel<8>, dim3(grid), dim3(PROBE_NT), 0, st, pa, na, pb, nb, chunk, never, out); break;
    case 16: hipLaunchKernelGGL(read_probe_kernel<16>, dim3(grid), dim3(PROBE_NT), 0, st, pa, na, pb, nb, chunk, never, out); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
