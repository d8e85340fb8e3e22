// Decode attention over a paged KV cache for gfx950 (MI355X): the per-partition pass for
// launches without copy-on-write, the scheduling word, and the split-K merges. The kernel
// itself and its design notes are in decode_kernel.h.
#include <mutex>
#include <vector>

#include "decode_kernel.h"

namespace pkv {

__global__ void sched_init_kernel(unsigned long long* sched) {
  if (threadIdx.x == 0) *sched = (unsigned long long)kSchedCookie << 32;
}

hipError_t launch_sched_init(unsigned long long* sched, hipStream_t stream) {
  hipLaunchKernelGGL(sched_init_kernel, dim3(1), dim3(64), 0, stream, sched);
  return hipGetLastError();
}

// Merge of the partitions of one (sequence, query head):
//   out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,   M = max_p m_p.
// 256 lanes: D/4 lanes cover a row with 16-byte loads and S = 1024/D slices take the
// partitions in turn (slice s gets p = s, s + S, ...). Each slice keeps a running (max, sum,
// accumulator), rescaled as its max grows, so every load of the partials is issued in one
// pass; the slices are then combined in slice order. The result is deterministic.
template <int D>
__global__ __launch_bounds__(256) void paged_decode_reduce_kernel(DecodeArgs a) {
  constexpr int LPR = D / 4;          // lanes per row
  constexpr int S = 256 / LPR;        // partition slices
  __shared__ float s_max[S];
  __shared__ float s_den[S];
  __shared__ float4 s_num[S][LPR];
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int cap = a.max_blocks << a.bs_log2;
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int nparts = L == 0 ? 1 : (L + a.part - 1) / a.part;
  if (nparts <= 1) return;
  const int sl = threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  const size_t base = ((size_t)b * a.num_q_heads + h) * a.pmax;
  const float* __restrict__ ml = a.ws_ml + base * 2;
  const float4* __restrict__ acc = reinterpret_cast<const float4*>(a.ws_acc + base * D) + c;

  float m = -INFINITY, den = 0.f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int p = sl; p < nparts; p += S) {
    const float mp = ml[2 * p];
    const float lp = ml[2 * p + 1];
    const float4 x = acc[(size_t)p * LPR];
    const float mn = fmaxf(m, mp);
    const float fo = m == -INFINITY ? 0.f : exp2f(m - mn);   // rescale of what came before
    const float fp = mp == -INFINITY ? 0.f : exp2f(mp - mn);  // weight of this partition
    den = den * fo + lp * fp;
    num.x = __builtin_fmaf(x.x, fp, num.x * fo);
    num.y = __builtin_fmaf(x.y, fp, num.y * fo);
    num.z = __builtin_fmaf(x.z, fp, num.z * fo);
    num.w = __builtin_fmaf(x.w, fp, num.w * fo);
    m = mn;
  }
  s_num[sl][c] = num;
  if (c == 0) {
    s_max[sl] = m;
    s_den[sl] = den;
  }
  __syncthreads();
  if (sl == 0) {
    float M = s_max[0];
#pragma unroll
    for (int i = 1; i < S; ++i) M = fmaxf(M, s_max[i]);
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
    float dt = 0.f;
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const float f = s_max[i] == -INFINITY ? 0.f : exp2f(s_max[i] - M);
      const float4 x = s_num[i][c];
      t.x = __builtin_fmaf(f, x.x, t.x);
      t.y = __builtin_fmaf(f, x.y, t.y);
      t.z = __builtin_fmaf(f, x.z, t.z);
      t.w = __builtin_fmaf(f, x.w, t.w);
      dt = __builtin_fmaf(f, s_den[i], dt);
    }
    const size_t o = ((size_t)b * a.num_q_heads + h) * D + c * 4;
    const bool ok = dt > 0.f;
    store_out(a.out, o + 0, ok ? t.x / dt : 0.f, a.out_dtype);
    store_out(a.out, o + 1, ok ? t.y / dt : 0.f, a.out_dtype);
    store_out(a.out, o + 2, ok ? t.z / dt : 0.f, a.out_dtype);
    store_out(a.out, o + 3, ok ? t.w / dt : 0.f, a.out_dtype);
  }
}


int resident_groups(const void* kernel, size_t lds) {
  struct Entry {
    const void* kernel;
    size_t lds;
    int device, groups;
  };
  static std::mutex mu;
  static std::vector<Entry> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (const Entry& e : cache)
      if (e.kernel == kernel && e.lds == lds && e.device == dev) return e.groups;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kDecodeThreads, lds) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  const int groups = per_cu * cus;
  std::lock_guard<std::mutex> lock(mu);
  cache.push_back({kernel, lds, dev, groups});
  return groups;
}

hipError_t launch_decode_partitions(const DecodeArgs& a, int kv_dtype, int head_dim, int group,
                                    hipStream_t stream, int* ticketed) {
  if (a.cow_src != nullptr)
    return launch_decode_partitions_cow(a, kv_dtype, head_dim, group, stream, ticketed);
  switch (kv_dtype) {
    case F32: return launch_d<F32, false>(a, head_dim, group, stream, ticketed);
    case F16: return launch_d<F16, false>(a, head_dim, group, stream, ticketed);
    case BF16: return launch_d<BF16, false>(a, head_dim, group, stream, ticketed);
    default: return hipErrorInvalidValue;
  }
}

// The same merge for sequences of a few partitions, one workgroup per sequence for all its
// query heads: D/16 lanes cover a head's row (16 columns each: four 16-byte loads per
// partition) and the workgroup takes 256/(D/16) heads at a time. A batch of short sequences
// then needs one small workgroup per sequence (a workgroup per row would mostly be dispatched
// to find nothing to do). Partitions are folded in ascending order with a running (max, sum,
// accumulator), rescaled as the max grows; the result is deterministic.
template <int D>
__global__ __launch_bounds__(256) void paged_decode_reduce_seq_kernel(DecodeArgs a) {
  constexpr int LPH = D / 16;         // lanes per head row
  constexpr int HPP = 256 / LPH;      // heads per pass of the workgroup
  const int b = blockIdx.x;
  const int cap = a.max_blocks << a.bs_log2;
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int nparts = L == 0 ? 1 : (L + a.part - 1) / a.part;
  if (nparts <= 1) return;
  const int c = threadIdx.x % LPH;
  for (int h = threadIdx.x / LPH; h < a.num_q_heads; h += HPP) {
    const size_t base = ((size_t)b * a.num_q_heads + h) * a.pmax;
    const float* __restrict__ ml = a.ws_ml + base * 2;
    const float4* __restrict__ acc = reinterpret_cast<const float4*>(a.ws_acc + base * D) + c * 4;
    float m = -INFINITY, den = 0.f;
    float4 num[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) num[i] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 2
    for (int p = 0; p < nparts; ++p) {
      const float mp = ml[2 * p];
      const float lp = ml[2 * p + 1];
      float4 x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = acc[(size_t)p * (D / 4) + i];
      const float mn = fmaxf(m, mp);
      const float fo = m == -INFINITY ? 0.f : exp2f(m - mn);   // rescale of what came before
      const float fp = mp == -INFINITY ? 0.f : exp2f(mp - mn);  // weight of this partition
      den = den * fo + lp * fp;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        num[i].x = __builtin_fmaf(x[i].x, fp, num[i].x * fo);
        num[i].y = __builtin_fmaf(x[i].y, fp, num[i].y * fo);
        num[i].z = __builtin_fmaf(x[i].z, fp, num[i].z * fo);
        num[i].w = __builtin_fmaf(x[i].w, fp, num[i].w * fo);
      }
      m = mn;
    }
    const bool ok = den > 0.f;
    float y[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y[4 * i + 0] = ok ? num[i].x / den : 0.f;
      y[4 * i + 1] = ok ? num[i].y / den : 0.f;
      y[4 * i + 2] = ok ? num[i].z / den : 0.f;
      y[4 * i + 3] = ok ? num[i].w / den : 0.f;
    }
    const size_t o = ((size_t)b * a.num_q_heads + h) * D + c * 16;
    if (a.out_dtype == F32) {
      float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + o);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = make_float4(y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]);
    } else {
      u32x4 w[2];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t lo = a.out_dtype == BF16 ? narrow_bits<BF16>(y[2 * i]) : narrow_bits<F16>(y[2 * i]);
        const uint32_t hi =
            a.out_dtype == BF16 ? narrow_bits<BF16>(y[2 * i + 1]) : narrow_bits<F16>(y[2 * i + 1]);
        w[i >> 2][i & 3] = lo | (hi << 16);
      }
      u32x4* dst = reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.out) + o);
      dst[0] = w[0];
      dst[1] = w[1];
    }
  }
}

// Partitions per sequence up to which the per-sequence merge is used.
constexpr int kSeqReduceMaxParts = 16;

hipError_t launch_decode_reduce(const DecodeArgs& a, int head_dim, hipStream_t stream) {
  if (a.pmax <= kSeqReduceMaxParts) {
    const dim3 grid((unsigned)a.num_seqs);
    switch (head_dim) {
      case 64: hipLaunchKernelGGL(paged_decode_reduce_seq_kernel<64>, grid, dim3(256), 0, stream, a); break;
      case 128: hipLaunchKernelGGL(paged_decode_reduce_seq_kernel<128>, grid, dim3(256), 0, stream, a); break;
      case 256: hipLaunchKernelGGL(paged_decode_reduce_seq_kernel<256>, grid, dim3(256), 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const dim3 grid(a.num_q_heads, a.num_seqs);
  switch (head_dim) {
    case 64: hipLaunchKernelGGL(paged_decode_reduce_kernel<64>, grid, dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(paged_decode_reduce_kernel<128>, grid, dim3(256), 0, stream, a); break;
    case 256: hipLaunchKernelGGL(paged_decode_reduce_kernel<256>, grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
