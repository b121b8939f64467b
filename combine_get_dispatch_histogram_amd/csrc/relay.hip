// relay.hip -- bookkeeping of the two-level relay on one GPU.
//
// "DeepEP Normal vs Low-Latency dual-mode analysis", normal-mode internode
// dispatch: a token crosses the network once per destination node (RDMA
// rank = rank / 8), lands in that node's RDMA buffer with its source
// metadata, and a forwarder copies it into the buffer of each of the
// node's ranks that wants it.  "Chapter 4  V1: layout, dispatch and
// combine", section 4.2: the internode handle adds RDMA prefixes and the
// source metadata.
//
// With the ranks as partitions of one GPU the relay is: notify over groups
// (notify.hip, group mode) -> this kernel -> pack into the group rows ->
// pack from the group rows into the ranks' rows (pack.hip, forwarding
// mode).  The kernel here records, for every group row, its source token
// and the row it takes in each of the group's 8 ranks, read from the
// direct dispatch's send_head (rank r's rows are in (source, token) order
// on both paths, so the forwarder's order is the same).
#include "device.h"
#include "kernels.h"

namespace miep {

// One thread per (token, group): 2 x 16-byte loads of the token's 8
// send_head entries of the group, 2 x 16-byte stores of the row's heads.
__global__ __launch_bounds__(256) void relay_meta_kernel(RelayMetaArgs a) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= a.N * a.G) return;
  const int64_t n = i / a.G;
  const int g = static_cast<int>(i - n * a.G);
  const int h = a.send_rdma_head[i];
  if (h < 0) return;
  const int64_t row = static_cast<int64_t>(a.rdma_off[g]) + h;
  if (row >= a.rdma_capacity) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(a.send_head + n * a.R + g * 8);
  const u32x4 lo = src[0], hi = src[1];
  u32x4* dst = reinterpret_cast<u32x4*>(a.send_nvl_head + row * 8);
  __builtin_nontemporal_store(lo, dst);
  __builtin_nontemporal_store(hi, dst + 1);
  __builtin_nontemporal_store(static_cast<int32_t>(n), a.rdma_src_idx + row);
}

hipError_t launch_relay_meta(const RelayMetaArgs& a, hipStream_t st) {
  const int64_t n = a.N * a.G;
  if (n == 0) return hipSuccess;
  if ((n + 255) / 256 > max_blocks(256)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(relay_meta_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace miep
