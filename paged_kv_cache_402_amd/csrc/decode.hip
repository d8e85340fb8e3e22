// Decode attention over a paged KV cache for gfx950 (MI355X).
//
// Pages cited:
//   P1 = openeuler.csdn.net/6ae29ebb40858c2d88170ea6.html (explainer, sections 1-9)
//   P2 = agent.csdn.net/6a744dae662f9a54cb99003e.html (article, sections 1-5)
//   P3 = aiknowledge.cn "2.2 PagedAttention 与 KV Cache 分页管理" (sections 2.2.1-2.2.13)
//
// The operation (P1 §4.2; P3 §2.2.3-§2.2.4): a sequence's keys and values sit in fixed-size
// physical blocks listed by its block table; the kernel reads them block by block through the
// table and computes ordinary softmax attention of the new token's query over all of them.
//
// Work decomposition (our design for gfx950; the pages give no kernel structure):
//   * one 256-lane workgroup per (KV head, sequence, context partition of `part` tokens);
//     grid x is the KV head, so with 8 KV heads every workgroup of one head runs on the same
//     XCD (workgroups are dealt to the 8 XCDs round-robin) and blocks shared by many
//     sequences (a common prompt prefix) stay in that XCD's L2;
//   * the G query rows of the GQA group are staged in LDS once, then held in registers;
//   * K pass: 8 (or 16) lanes own one token row, each lane loads 16-byte vectors of it, takes
//     the dot product with its slice of each query row (v_dot2 for 16-bit data), and a DPP
//     butterfly inside the lane group finishes the sum; the scores of the partition go to LDS;
//     the block id is resolved once per group of tokens from the table (a scalar load);
//   * exact softmax inside the partition: max over the partition, then exp2 and the sum;
//   * V pass: 16 lanes own one token row, each lane accumulates p * v for its 8 (or 4)
//     columns and every head of the group in fp32;
//   * the lane groups, then the 4 waves, are combined through LDS; a sequence that fits one
//     partition gets its output row directly, longer ones leave (max, sum, accumulator)
//     partials that a second kernel merges in partition order (deterministic split-K).
// Every loop bound is uniform; loads of a step are issued together before any use so each
// wave keeps 8 x 16-byte vectors (8 KiB per wave) in flight.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace pkv {

template <int DT, int D, int G>
struct Cfg {
  static constexpr int EB = Elem<DT>::bytes;
  static constexpr int PER16 = Elem<DT>::per16;
  static constexpr int RB = D * EB;                    // bytes of one token row of one head
  static constexpr int C = RB / 16;                    // 16-byte vectors per row
  static constexpr int LK = C <= 16 ? 8 : 16;          // lanes per token row, K pass
  static constexpr int NLK = C / LK;                   // vectors per lane per row, K pass
  static constexpr int TK = 64 / LK;                   // token rows per wave step, K pass
  static constexpr int UK = NLK >= 8 ? 1 : 8 / NLK;    // wave steps per load round, K pass
  static constexpr int LV = C < 16 ? C : 16;           // lanes per token row, V pass
  static constexpr int NLV = C / LV;
  static constexpr int TV = 64 / LV;
  static constexpr int UV = NLV >= 8 ? 1 : 8 / NLV;
  static constexpr int ACC = NLV * PER16;              // accumulators per lane per head
  static_assert(C >= 8 && C % LK == 0 && C % LV == 0, "row must be a multiple of 128 bytes");
  static_assert(TK <= 8 && TV <= 8, "a wave step must stay inside one block of >= 8 tokens");
};

template <int N> __device__ __forceinline__ void lds_store_n(float* dst, const float* v) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 4)
      *reinterpret_cast<float4*>(dst + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
  } else if constexpr (N == 2) {
    *reinterpret_cast<float2*>(dst) = make_float2(v[0], v[1]);
  } else {
    dst[0] = v[0];
  }
}
template <int N> __device__ __forceinline__ void lds_load_n(const float* src, float* v) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      float4 x = *reinterpret_cast<const float4*>(src + i);
      v[i] = x.x; v[i + 1] = x.y; v[i + 2] = x.z; v[i + 3] = x.w;
    }
  } else if constexpr (N == 2) {
    float2 x = *reinterpret_cast<const float2*>(src);
    v[0] = x.x; v[1] = x.y;
  } else {
    v[0] = src[0];
  }
}

__device__ __forceinline__ void store_out(void* out, size_t idx, float y, int out_dtype) {
  if (out_dtype == F32) {
    reinterpret_cast<float*>(out)[idx] = y;
  } else if (out_dtype == BF16) {
    reinterpret_cast<uint16_t*>(out)[idx] = (uint16_t)narrow_bits<BF16>(y);
  } else {
    reinterpret_cast<uint16_t*>(out)[idx] = (uint16_t)narrow_bits<F16>(y);
  }
}

template <int DT, int D, int G>
__global__ __launch_bounds__(kDecodeThreads) void paged_decode_partition_kernel(DecodeArgs a) {
  using K = Cfg<DT, D, G>;
  constexpr int NT = kDecodeThreads, NW = kDecodeWaves;
  extern __shared__ __align__(16) unsigned char smem[];

  const int kvh = blockIdx.x;
  const int b = blockIdx.y;
  const int pi = blockIdx.z;
  const int cap = a.max_blocks << a.bs_log2;
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int nparts = L == 0 ? 1 : (L + a.part - 1) / a.part;
  if (pi >= nparts) return;
  const int t0 = pi * a.part;
  const int n = min(L - t0, a.part);  // tokens of this partition (0 only when L == 0)

  const int bs_mask = (1 << a.bs_log2) - 1;
  const int32_t* __restrict__ trow = a.block_tables + (size_t)b * a.max_blocks;
  const size_t head_bytes = ((size_t)1 << a.bs_log2) * K::RB;     // one (block, head) tile
  const size_t block_bytes = head_bytes * a.num_kv_heads;         // one block, all heads
  const unsigned char* kbase = (const unsigned char*)a.k_cache + kvh * head_bytes;
  const unsigned char* vbase = (const unsigned char*)a.v_cache + kvh * head_bytes;

  const int sc_floats = max(a.part * G, NW * G * D);
  float* s_sc = reinterpret_cast<float*>(smem);                    // [part][G] scores / probs
  u32x4* s_q = reinterpret_cast<u32x4*>(smem + (size_t)sc_floats * 4);  // [G][C]
  float* s_red = reinterpret_cast<float*>(smem + (size_t)sc_floats * 4 + G * K::RB);  // [2][NW][G]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- stage the query group in LDS (heads kvh*G .. kvh*G+G-1 are contiguous) ----
  const unsigned char* qsrc =
      (const unsigned char*)a.q + ((size_t)b * a.num_q_heads + (size_t)kvh * G) * K::RB;
  for (int i = tid; i < G * K::C; i += NT) s_q[i] = load16(qsrc + (size_t)i * 16);
  __syncthreads();

  const int kr = lane / K::LK;  // token row inside a K step
  const int kc = lane % K::LK;  // this lane's vectors: kc, kc+LK, ...
  u32x4 qv[G][K::NLK];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < K::NLK; ++i) qv[g][i] = s_q[g * K::C + kc + i * K::LK];

  // ---- K pass: scores (base-2 units) of every token of the partition -> LDS ----
  float m[G];
#pragma unroll
  for (int g = 0; g < G; ++g) m[g] = -INFINITY;
  const int ngk = (n + K::TK - 1) / K::TK;
  for (int g0 = wave; g0 < ngk; g0 += NW * K::UK) {
    u32x4 kv[K::UK][K::NLK];
    bool okb[K::UK];
#pragma unroll
    for (int u = 0; u < K::UK; ++u) {
      const int gi = g0 + u * NW;
      okb[u] = false;
      if (gi < ngk) {
        const int tok = t0 + gi * K::TK;
        int blk = trow[tok >> a.bs_log2];
        okb[u] = (unsigned)blk < (unsigned)a.num_blocks;
        blk = okb[u] ? blk : 0;  // an invalid entry reads block 0 and is masked below
        const unsigned char* p = kbase + (size_t)blk * block_bytes +
                                 (size_t)((tok & bs_mask) + kr) * K::RB + kc * 16;
#pragma unroll
        for (int i = 0; i < K::NLK; ++i) kv[u][i] = load16(p + i * K::LK * 16);
      }
    }
#pragma unroll
    for (int u = 0; u < K::UK; ++u) {
      const int gi = g0 + u * NW;
      if (gi < ngk) {
        float s[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float acc = 0.f;
#pragma unroll
          for (int i = 0; i < K::NLK; ++i) acc = dot16<DT>(qv[g][i], kv[u][i], acc);
          s[g] = group_sum<K::LK>(acc) * a.scale_log2;
        }
        const int tl = gi * K::TK + kr;
        const bool valid = okb[u] && tl < n;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          s[g] = valid ? s[g] : -INFINITY;
          m[g] = fmaxf(m[g], s[g]);
        }
        if (kc == 0 && tl < n) lds_store_n<G>(s_sc + tl * G, s);
      }
    }
  }

  // ---- partition max: lanes of one row agree; combine rows, then waves ----
#pragma unroll
  for (int g = 0; g < G; ++g) m[g] = xor_max_from<K::LK>(m[g]);
  if (lane == 0) lds_store_n<G>(s_red + wave * G, m);
  __syncthreads();
  float mg[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float x = s_red[g];
#pragma unroll
    for (int w = 1; w < NW; ++w) x = fmaxf(x, s_red[w * G + g]);
    mg[g] = x == -INFINITY ? 0.f : x;  // nothing valid: every weight becomes exp2(-inf) = 0
  }

  // ---- probabilities p = 2^(s - max) in place, and this lane's share of their sum ----
  float l[G];
#pragma unroll
  for (int g = 0; g < G; ++g) l[g] = 0.f;
  for (int t = tid; t < n; t += NT) {
    float v[G];
    lds_load_n<G>(s_sc + t * G, v);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      v[g] = exp2f(v[g] - mg[g]);
      l[g] += v[g];
    }
    lds_store_n<G>(s_sc + t * G, v);
  }
  __syncthreads();

  // ---- V pass: acc[g][:] += p[g] * v over the partition ----
  const int vr = lane / K::LV;
  const int vc = lane % K::LV;
  float acc[G][K::ACC];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < K::ACC; ++e) acc[g][e] = 0.f;
  const int ngv = (n + K::TV - 1) / K::TV;
  for (int g0 = wave; g0 < ngv; g0 += NW * K::UV) {
    u32x4 vv[K::UV][K::NLV];
    bool okb[K::UV];
#pragma unroll
    for (int u = 0; u < K::UV; ++u) {
      const int gi = g0 + u * NW;
      okb[u] = false;
      if (gi < ngv) {
        const int tok = t0 + gi * K::TV;
        int blk = trow[tok >> a.bs_log2];
        okb[u] = (unsigned)blk < (unsigned)a.num_blocks;
        blk = okb[u] ? blk : 0;
        const unsigned char* p = vbase + (size_t)blk * block_bytes +
                                 (size_t)((tok & bs_mask) + vr) * K::RB + vc * 16;
#pragma unroll
        for (int i = 0; i < K::NLV; ++i) vv[u][i] = load16(p + i * K::LV * 16);
      }
    }
#pragma unroll
    for (int u = 0; u < K::UV; ++u) {
      const int gi = g0 + u * NW;
      const int tl = gi * K::TV + vr;
      // tokens past the sequence end may hold anything (even NaN): skip, never multiply by 0
      if (gi < ngv && okb[u] && tl < n) {
        float pg[G];
        lds_load_n<G>(s_sc + tl * G, pg);
#pragma unroll
        for (int i = 0; i < K::NLV; ++i) {
          float f[K::PER16];
          widen<DT>(vv[u][i], f);
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < K::PER16; ++e)
              acc[g][i * K::PER16 + e] = __builtin_fmaf(pg[g], f[e], acc[g][i * K::PER16 + e]);
        }
      }
    }
  }

  // ---- combine: rows inside each wave (shuffles), then the waves (LDS) ----
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int e = 0; e < K::ACC; ++e) acc[g][e] = xor_sum_from<K::LV>(acc[g][e]);
    l[g] = xor_sum_from<1>(l[g]);
  }
  __syncthreads();  // every wave is done reading probabilities from s_sc
  float* s_acc = s_sc;  // [NW][G][D]
  if (vr == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < K::NLV; ++i)
        lds_store_n<K::PER16>(s_acc + (wave * G + g) * D + (i * K::LV + vc) * K::PER16,
                              &acc[g][i * K::PER16]);
  }
  if (lane == 0) lds_store_n<G>(s_red + NW * G + wave * G, l);
  __syncthreads();

  const bool single = nparts == 1;
  for (int idx = tid; idx < G * D; idx += NT) {
    const int g = idx / D;
    const int d = idx - g * D;
    float x = s_acc[g * D + d];
    float lt = s_red[NW * G + g];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      x += s_acc[(w * G + g) * D + d];
      lt += s_red[NW * G + w * G + g];
    }
    const int h = kvh * G + g;
    if (single) {
      const float y = lt > 0.f ? x / lt : 0.f;
      store_out(a.out, ((size_t)b * a.num_q_heads + h) * D + d, y, a.out_dtype);
    } else {
      const size_t slot = ((size_t)b * a.num_q_heads + h) * a.pmax + pi;
      a.ws_acc[slot * D + d] = x;
      if (d == 0) {
        float mm = s_red[g];
#pragma unroll
        for (int w = 1; w < NW; ++w) mm = fmaxf(mm, s_red[w * G + g]);
        a.ws_ml[slot * 2] = mm == -INFINITY ? 0.f : mm;
        a.ws_ml[slot * 2 + 1] = lt;
      }
    }
  }
}

// Merge of the partitions of one (sequence, query head), in partition order:
//   out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,   M = max_p m_p.
template <int D>
__global__ __launch_bounds__(D) void paged_decode_reduce_kernel(DecodeArgs a) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  const int cap = a.max_blocks << a.bs_log2;
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int nparts = L == 0 ? 1 : (L + a.part - 1) / a.part;
  if (nparts <= 1) return;
  const size_t base = ((size_t)b * a.num_q_heads + h) * a.pmax;
  const float* __restrict__ ml = a.ws_ml + base * 2;
  const float* __restrict__ acc = a.ws_acc + base * D + d;
  float M = -INFINITY;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, ml[2 * p]);
  float num = 0.f, den = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float w = exp2f(ml[2 * p] - M);
    den = __builtin_fmaf(w, ml[2 * p + 1], den);
    num = __builtin_fmaf(w, acc[(size_t)p * D], num);
  }
  const float y = den > 0.f ? num / den : 0.f;
  store_out(a.out, ((size_t)b * a.num_q_heads + h) * D + d, y, a.out_dtype);
}

size_t decode_lds_bytes(int kv_dtype, int head_dim, int group, int part) {
  const int eb = kv_dtype == F32 ? 4 : 2;
  const size_t sc = (size_t)(part * group > kDecodeWaves * group * head_dim
                                 ? part * group
                                 : kDecodeWaves * group * head_dim);
  return sc * 4 + (size_t)group * head_dim * eb + 2 * kDecodeWaves * group * 4;
}

template <int DT, int D, int G>
static hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.num_kv_heads, a.num_seqs, a.pmax);
  const size_t lds = decode_lds_bytes(DT, D, G, a.part);
  hipLaunchKernelGGL((paged_decode_partition_kernel<DT, D, G>), grid, dim3(kDecodeThreads), lds,
                     stream, a);
  return hipGetLastError();
}

template <int DT, int D>
static hipError_t launch_g(const DecodeArgs& a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_t<DT, D, 1>(a, stream);
    case 2: return launch_t<DT, D, 2>(a, stream);
    case 4: return launch_t<DT, D, 4>(a, stream);
    case 8:
      if constexpr (D <= 128) return launch_t<DT, D, 8>(a, stream);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
static hipError_t launch_d(const DecodeArgs& a, int head_dim, int group, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_g<DT, 64>(a, group, stream);
    case 128: return launch_g<DT, 128>(a, group, stream);
    case 256: return launch_g<DT, 256>(a, group, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_partitions(const DecodeArgs& a, int kv_dtype, int head_dim, int group,
                                    hipStream_t stream) {
  switch (kv_dtype) {
    case F32: return launch_d<F32>(a, head_dim, group, stream);
    case F16: return launch_d<F16>(a, head_dim, group, stream);
    case BF16: return launch_d<BF16>(a, head_dim, group, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_reduce(const DecodeArgs& a, int head_dim, hipStream_t stream) {
  const dim3 grid(a.num_q_heads, a.num_seqs);
  switch (head_dim) {
    case 64: hipLaunchKernelGGL(paged_decode_reduce_kernel<64>, grid, dim3(64), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(paged_decode_reduce_kernel<128>, grid, dim3(128), 0, stream, a); break;
    case 256: hipLaunchKernelGGL(paged_decode_reduce_kernel<256>, grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
