// Boundary state view (LongSpark paper page, Fig. 2 (b): one of the views is a
// state taken from the target at the accepted boundary).  After verification
// tau[c] positions of the verified block are committed; the boundary is the
// newest of them, row tau[c] - 1 of the block's [B+1, H] states.  The view is
// a copy of that row, bit for bit, chosen on the device from tau so that it
// chains after verification without a host round trip.
//
// One workgroup per sequence; 16-byte pieces when the rows allow it, else
// element copies.  tau outside [1, B+1] is clamped and flagged.
#include "common.hpp"
#include "launch.hpp"

namespace ls {
namespace {

constexpr int kThreads = 256;

template <int E>  // element size in bytes
__global__ __launch_bounds__(kThreads) void boundary_gather(
    const uint8_t* __restrict__ hidden, const int32_t* __restrict__ tau, uint8_t* __restrict__ out,
    int32_t* __restrict__ err_flag, int B1, int H, int vec) {
  const int c = blockIdx.x;
  int t = tau[c];
  if (t < 1 || t > B1) {
    if (threadIdx.x == 0 && err_flag != nullptr) atomicOr(err_flag, 1);
    t = t < 1 ? 1 : B1;
  }
  const int64_t row_bytes = int64_t(H) * E;
  const uint8_t* src = hidden + (int64_t(c) * B1 + (t - 1)) * row_bytes;
  uint8_t* dst = out + int64_t(c) * row_bytes;
  if (vec) {
    for (int64_t p = threadIdx.x; p < row_bytes / 16; p += kThreads)
      reinterpret_cast<uint4*>(dst)[p] = reinterpret_cast<const uint4*>(src)[p];
  } else if (E == 4) {
    for (int64_t p = threadIdx.x; p < H; p += kThreads)
      reinterpret_cast<uint32_t*>(dst)[p] = reinterpret_cast<const uint32_t*>(src)[p];
  } else {
    for (int64_t p = threadIdx.x; p < H; p += kThreads)
      reinterpret_cast<uint16_t*>(dst)[p] = reinterpret_cast<const uint16_t*>(src)[p];
  }
}

}  // namespace

ls_status launch_boundary(const ls_dims& d, const void* hidden, int32_t H, const int32_t* tau,
                          void* out, int32_t* err_flag, hipStream_t stream) {
  const int esz = d.dtype == LS_BF16 ? 2 : 4;
  // 16-byte pieces need 16-byte rows and 16-byte aligned buffers
  const int vec = (int64_t(H) * esz) % 16 == 0 && (uintptr_t(hidden) & 15) == 0 &&
                  (uintptr_t(out) & 15) == 0;
  const auto* src = static_cast<const uint8_t*>(hidden);
  auto* dst = static_cast<uint8_t*>(out);
  if (esz == 2)
    hipLaunchKernelGGL(boundary_gather<2>, dim3(d.C), dim3(kThreads), 0, stream, src, tau, dst,
                       err_flag, d.B + 1, H, vec);
  else
    hipLaunchKernelGGL(boundary_gather<4>, dim3(d.C), dim3(kThreads), 0, stream, src, tau, dst,
                       err_flag, d.B + 1, H, vec);
  return hipGetLastError() == hipSuccess ? LS_OK : LS_ERR_HIP;
}

}  // namespace ls
