// Cache write (slot mapping) and copy-on-write block copy for gfx950. Both are bit copies in
// 16-byte vectors; neither converts data.
//
// Pages cited:
//   P1 = openeuler.csdn.net/6ae29ebb40858c2d88170ea6.html (explainer, sections 1-9)
//   P2 = agent.csdn.net/6a744dae662f9a54cb99003e.html (article, sections 1-5)
//   P3 = aiknowledge.cn "2.2 PagedAttention 与 KV Cache 分页管理" (sections 2.2.1-2.2.13)
//
// Cache write (P1 §4.3; P3 §2.2.2-§2.2.3): the K and V rows of each new token go to the slot
// the block manager reserved: block slot / block_size, offset slot % block_size.
// Block copy (P1 §6.2; P2 §2.2): a write into a shared block first duplicates that one block,
// all heads and slots, K and V.
#include "common.h"
#include "launch.h"

namespace pkv {

// One workgroup per (token, 256 vectors of its [Hkv][D] rows).
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(CacheWriteArgs a) {
  const int t = blockIdx.x;
  const int vecs_per_row = a.row_bytes / 16;
  const int c = blockIdx.y * 256 + threadIdx.x;
  if (c >= a.num_kv_heads * vecs_per_row) return;
  const int slot = a.slots[t];
  const long long nslots = (long long)a.num_blocks << a.bs_log2;
  if (slot < 0 || slot >= nslots) return;  // negative: skip; past the pool: ignored
  const int h = c / vecs_per_row;
  const int v = c - h * vecs_per_row;
  const int blk = slot >> a.bs_log2;
  const int off = slot & ((1 << a.bs_log2) - 1);
  const size_t src = ((size_t)t * a.num_kv_heads + h) * a.row_bytes + (size_t)v * 16;
  const size_t dst =
      (((size_t)blk * a.num_kv_heads + h) << a.bs_log2 | (size_t)off) * a.row_bytes + (size_t)v * 16;
  store16((unsigned char*)a.k_cache + dst, load16((const unsigned char*)a.k + src));
  store16((unsigned char*)a.v_cache + dst, load16((const unsigned char*)a.v + src));
}

hipError_t launch_reshape_and_cache(const CacheWriteArgs& a, hipStream_t stream) {
  const int vecs = a.num_kv_heads * (a.row_bytes / 16);
  const dim3 grid(a.num_tokens, (vecs + 255) / 256);
  hipLaunchKernelGGL(reshape_and_cache_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

// One workgroup per (pair, 4096 vectors of the block); each lane moves 16 B of K and of V per
// step and issues the loads of kCopyUnroll steps before their stores (src and dst are
// different blocks, so the loads never read what the stores write).
constexpr int kCopyVecsPerGroup = 4096;
constexpr int kCopyUnroll = 4;

__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyBlocksArgs a) {
  const int pr = blockIdx.x;
  const int src = a.pairs[2 * pr];
  const int dst = a.pairs[2 * pr + 1];
  if ((unsigned)src >= (unsigned)a.num_blocks || (unsigned)dst >= (unsigned)a.num_blocks) return;
  const int64_t nvec = a.block_bytes / 16;
  const int64_t v0 = (int64_t)blockIdx.y * kCopyVecsPerGroup;
  const int64_t v1 = v0 + kCopyVecsPerGroup < nvec ? v0 + kCopyVecsPerGroup : nvec;
  const size_t so = (size_t)src * a.block_bytes, dof = (size_t)dst * a.block_bytes;
  const unsigned char* ks = (const unsigned char*)a.k_cache + so;
  const unsigned char* vs = (const unsigned char*)a.v_cache + so;
  unsigned char* kd = (unsigned char*)a.k_cache + dof;
  unsigned char* vd = (unsigned char*)a.v_cache + dof;
  for (int64_t i0 = v0 + threadIdx.x; i0 < v1; i0 += 256 * kCopyUnroll) {
    u32x4 x[kCopyUnroll], y[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = i0 + u * 256;
      if (i < v1) {
        x[u] = load16(ks + i * 16);
        y[u] = load16(vs + i * 16);
      }
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = i0 + u * 256;
      if (i < v1) {
        store16(kd + i * 16, x[u]);
        store16(vd + i * 16, y[u]);
      }
    }
  }
}

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream) {
  const int64_t nvec = a.block_bytes / 16;
  const dim3 grid(a.num_pairs, (unsigned)((nvec + kCopyVecsPerGroup - 1) / kCopyVecsPerGroup));
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
